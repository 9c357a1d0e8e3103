// Internal declarations shared by the kd HIP sources (not part of the C ABI).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "kd.h"

namespace kd {

void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
// Checks hipGetLastError after a launch; sets the message and returns KD_ERR_HIP on failure.
kd_status check_launch(const char* what);

#define KD_REQUIRE(cond, code, ...)  \
  do {                               \
    if (!(cond)) {                   \
      ::kd::set_error(__VA_ARGS__);  \
      return (code);                 \
    }                                \
  } while (0)

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Quads of 4 blocks (128 elements) along k.
__host__ __device__ inline int n_quads(int k) { return ceil_div(k, 128); }
__host__ __device__ inline int n_rowgroups(int n_out) { return ceil_div(n_out, 16); }

// ---- device helpers -------------------------------------------------------------------
__device__ inline uint32_t pack4b(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
         ((uint32_t)(d & 0xFF) << 24);
}

// Activation quantiser on one 32-element block v[0..31]: a = max|v_i|; d = a / 127 (IEEE fp32
// division; 0 if a == 0); q_i = round-half-away(v_i / d) clamped to [-127, 127].  Codes are
// stored in the tiled activation layout (dst_block = row base + q*128 + j*8; group g's eight
// codes P_g = {4g..4g+3, 4g+16..4g+19} at dst_block + 32 g) and the scale at *d_out.
__device__ inline void quant32(const float* v, int8_t* dst_block, float* d_out) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float dd = amax / 127.0f;
  int c[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int qv = 0;
    if (amax != 0.0f) {
      qv = (int)roundf(v[i] / dd);
      qv = qv > 127 ? 127 : (qv < -127 ? -127 : qv);
    }
    c[i] = qv;
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint2 w;
    w.x = pack4b(c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]);
    w.y = pack4b(c[4 * g + 16], c[4 * g + 17], c[4 * g + 18], c[4 * g + 19]);
    *reinterpret_cast<uint2*>(dst_block + g * 32) = w;
  }
  *d_out = dd;
}

// DPP read of lane CTRL-permuted x within each 16-lane row (a VALU operand, where a shuffle
// goes through the LDS crossbar).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Sum and maximum over each aligned group of 8 lanes, the same value in all 8 (every lane of
// the group must be active): lane ^ 1, lane ^ 2, then the mirrored lane of the half row, which
// holds the other quad's partial.  Each step combines the same two partials as the xor
// butterfly over masks 1, 2, 4, so the results are equal bit for bit.
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  return x;
}
__device__ __forceinline__ float group8_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  return x;
}

// The same quantiser with a block spread over 8 consecutive lanes (lane sub = tid % 8 holds
// elements [4 sub, 4 sub + 4) in v).  Every lane of the group must execute it (shuffles);
// stores happen only if `store`.  Codes and scale equal quant32's for the same 32 values
// (max is exact and order-free; each code is computed alone).
__device__ inline void quant4_lane8(float4 v, int sub, bool store, int8_t* dst_block, float* d_out) {
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  amax = group8_max(amax);
  const float dd = amax / 127.0f;
  int c[4] = {0, 0, 0, 0};
  if (amax != 0.0f) {
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int qv = (int)roundf(e[i] / dd);
      c[i] = qv > 127 ? 127 : (qv < -127 ? -127 : qv);
    }
  }
  if (store) {
    // elements 4 sub .. 4 sub + 3: group (sub & 3), first half if sub < 4 else second half
    *reinterpret_cast<uint32_t*>(dst_block + 32 * (sub & 3) + (sub >> 2) * 4) = pack4b(c[0], c[1], c[2], c[3]);
    if (sub == 0) *d_out = dd;
  }
}

__device__ inline float4 f4_add(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }

__device__ inline float wave_sum(float v) {
  // xor butterfly: every lane ends with the same value (fp add is commutative).
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Maximum over the 64 lanes, the same value in every lane (exact in any order): DPP within
// each 16-lane row (lane ^ 1, lane ^ 2, the mirrored lane of the half row, of the row), then
// the four row maxima read from lanes 0, 16, 32, 48.  Call from uniform control flow.
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// cos/sin of the NEOX RoPE angle pos * base^(-2i/hd), evaluated in fp64, rounded to fp32.
__device__ inline float2 rope_cs(int pos, int i, int hd, double base) {
  const double theta = (double)pos * pow(base, -2.0 * (double)i / (double)hd);
  double s, c;
  sincos(theta, &s, &c);
  return make_float2((float)c, (float)s);
}

// fp32 -> FP8 E4M3 code (OCP layout: sign, 4 exponent bits with bias 7, 3 mantissa bits, no
// infinities, 0x7F / 0xFF NaN): nearest, ties to the even code; magnitudes past 448 (the
// largest finite value) saturate to it; NaN -> 0x7F with its sign.  Integer rounding of the
// fp32 mantissa for normal codes; subnormal codes (|x| < 2^-6) are |x| 2^9 rounded to even.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t c;
  if (a != a) {
    c = 0x7Fu;
  } else if (a >= 448.0f) {
    c = 0x7Eu;
  } else if (a < 0.015625f) {
    c = (uint32_t)rintf(a * 512.0f);  // 0 .. 8; 8 is 2^-6, the first normal code
  } else {
    const uint32_t au = __float_as_uint(a);
    const uint32_t e = (au >> 23) - 120u;  // biased E4M3 exponent, 1 .. 15
    const uint32_t m = au & 0x7FFFFFu;
    uint32_t r = m >> 20;
    const uint32_t rem = m & 0xFFFFFu;
    r += (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ? 1u : 0u;
    c = (e << 3) + r;  // a mantissa carry moves to the next exponent
  }
  return sign | c;
}

// ---- buffer loads ----------------------------------------------------------------------
// Raw (stride 0) buffer descriptors: an offset at or past num_records reads as zero without
// touching memory, which masks out-of-range lanes without a branch.
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every buffer the kernels read

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// AUX = 2: non-temporal (data streamed once) on gfx950.
template <int AUX>
__device__ __forceinline__ int4 buf16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
  return make_int4(v.x, v.y, v.z, v.w);
}
template <int AUX>
__device__ __forceinline__ uint2 buf8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
  return make_uint2((uint32_t)v.x, (uint32_t)v.y);
}
template <int AUX>
__device__ __forceinline__ uint32_t buf4u(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
}
__device__ __forceinline__ float buf4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// ---- launchers used by the step driver (arguments already validated) -------------------
int norm_max_len();
void launch_act_quant(const float* x, int B, int k, int ldx, int8_t* qs, float* d, hipStream_t st);
// Fused RMSNorm (optionally with a residual add) + activation quantiser.  If r != nullptr:
// x1 = x + r is written to x1_out.  y = rmsnorm(x or x1) is written to y_out if non-null.
// The quantised y goes to (qs, d) if qs != nullptr.
void launch_norm_quant(const float* x, const float* r, const float* g, int B, int n, float eps,
                       float* x1_out, float* y_out, int8_t* qs, float* d, hipStream_t st);

// Row maps for grouped (MoE) products: output row j of group e reads activation row
// act_row[e*16 + j] and writes output row out_row[e*16 + j], j < count[e].
struct RowMap {
  const int32_t* count;    // [n_groups]
  const int32_t* act_row;  // [n_groups * 16]
  const int32_t* out_row;  // [n_groups * 16]
  int n_groups;
  long long w_group_tiles;  // tiles between consecutive groups' weights
  int act_rows;             // rows of the activation buffer the act_row entries index
};

// Whether a Q8_0/Q4_0 matrix fits the product (k <= mmvq_max_k(), tiled arrays < 2 GiB).
bool mmvq_weight_fits(int fmt, int n_out, int k);
bool mmvq_fmt_ok(int fmt, int k);     // a quantised weight format, k a multiple of its block
bool mmvq_swiglu_fits(int k);         // the SwiGLU product's LDS at this k fits a CU
int mmvq_max_k();
// mo_y / mo_p / mo_K (plain products only): y is a MoE layer's output, the rank-order sum
// of the experts' rows mo_y [B K][n_out] weighted by mo_p [B][K], plus W x (the shared
// expert's down product): per element, an fma chain over k from 0, then + (W x).
void launch_mmvq(const kd_weight& W, const int8_t* xq, const float* xd, int B, float* y, int ldy,
                 hipStream_t st, const RowMap* map = nullptr, int32_t* debug_S = nullptr,
                 const float* mo_y = nullptr, const float* mo_p = nullptr, int mo_K = 0);

// Per-row cache addresses and positions of one layer, passed by value as a kernel argument
// (B <= 16 rows: no host-to-device copy and no synchronisation per step).
struct RowCaches {
  void* k[KD_MAX_B];
  void* v[KD_MAX_B];
  int32_t pos[KD_MAX_B];
};

// Fused products.  SwiGLU: W is the [2F, d] gate/up matrix interleaved in blocks of 32 rows
// (gate rows 32m.., then up rows 32m..); writes the quantised silu(gate) * up rows [B][F].
// With a row map (grouped experts): W holds each group's interleaved [2F, d] block, and
// output row j of group e goes to row out_row[e*16 + j] of (out_qs, out_d).
// Grouped (map): X, when given, is an extra matrix of whole groups' rows (the shared
// expert's interleaved gate/up, its n_out a multiple of W.n_out, same format and k) applied to
// all B rows in the same launch, its SwiGLU rows going to x_qs / x_qd (X.n_out / 2 columns);
// only when mmvq_swiglu_merges(W, X).
void launch_mmvq_swiglu(const kd_weight& W, const int8_t* xq, const float* xd, int B, int8_t* out_qs, float* out_d,
                        hipStream_t st, const float* norm_ss = nullptr, int norm_n = 0, float norm_eps = 0.0f,
                        const RowMap* map = nullptr, const kd_weight* X = nullptr, int8_t* x_qs = nullptr,
                        float* x_qd = nullptr);
bool mmvq_swiglu_merges(const kd_weight& W, const kd_weight& X);
// O-style product whose epilogue adds the residual and starts the next RMSNorm: x1 = res + W x
// (x1 may not alias res), Q8 codes of x1 * gain with per-block scales, and the per-block sums
// of squares ss [B][n_out / 32] that launch_mmvq_swiglu's norm_ss turns into 1/rms.
constexpr int kNormFuseMax = 4096;  // longest row whose block sums the consumer's 8 lanes hold
void launch_mmvq_resnorm(const kd_weight& W, const int8_t* xq, const float* xd, int B, const float* res, int ld,
                         const float* gain, float* x1, int8_t* out_qs, float* out_d, float* ss, hipStream_t st);
// RoPE: W is wqkv with each head's rows in pair order (i, i + hd/2 adjacent); writes the
// rotated q rows to q (stride ldq) and the rotated k and the v rows (fp16, or E4M3 codes when
// kv_fp8) at each row's position in its caches; cs is the step's cos/sin table.
// cs == nullptr: the angles are evaluated in the epilogue (rope_base), same values.
void launch_mmvq_rope(const kd_weight& W, const int8_t* xq, const float* xd, int B, float* q, int ldq, int H, int G,
                      int hd, const float* cs, float rope_base, const RowCaches& rc, int capacity, hipStream_t st,
                      const float* norm_ss = nullptr, int norm_n = 0, float norm_eps = 0.0f, bool kv_fp8 = false);

// cos/sin table [B][hd/2][2] fp32 from per-row positions (angles in fp64).
void launch_rope_table(const RowCaches& rc, int B, int hd, float base, float* cs, hipStream_t st);
// QK-norm first when q_norm / k_norm (per-head gains [hd]) are given.
// Rotates q (in place, rows of qkv with stride ldqkv) and k, rounds k and v to fp16 and
// stores them at each row's position (append) or only rotates (q and k heads).  cs is the
// per-step table, or null to evaluate cos/sin inline with the same fp64 expression.
// kv_fmt (kd_kv_format): the caches hold fp16 values, FP8 E4M3 codes (f32_to_e4m3) or int8 rows
// (kv_q8_row_bytes per (head, position): Q8_0 blocks, see q8_store_pair).
void launch_rope_append(float* qkv, int ldqkv, int B, int H, int G, int hd, const float* cs,
                        const RowCaches& rc, int capacity, bool append, hipStream_t st, float base,
                        const float* q_norm = nullptr, const float* k_norm = nullptr, float eps = 0.0f,
                        int kv_fmt = KD_KV_F16);
void launch_kv_append(const float* k, const float* v, int B, int G, int hd, const RowCaches& rc, int capacity,
                      hipStream_t st, int kv_fmt = KD_KV_F16);
// Bytes of one cached (KV head, position) row of an int8 cache: hd codes, hd/32 fp16 scales,
// zero padding to hd + 16.
__host__ __device__ constexpr int kv_q8_row_bytes(int hd) { return hd + 16; }
// Bytes between consecutive positions of one KV head's row stream, per cache format.
__host__ __device__ constexpr int kv_row_bytes(int kv_fmt, int hd) {
  return kv_fmt == KD_KV_Q8_0 ? kv_q8_row_bytes(hd) : kv_fmt == KD_KV_FP8_E4M3 ? hd : 2 * hd;
}

struct FaPlan {
  int B, H, G, hd;
  int n_items;                        // total (row, split) items
  int32_t split_off[KD_MAX_B + 1];    // prefix sums of splits per row
  int32_t chunk[KD_MAX_B];            // keys per split of each row
  int32_t t_kv[KD_MAX_B];             // keys attended by each row
  // Row groups that share one pass over a cache (set by launch_fa from the cache pointers):
  // consecutive rows of one cache with the same chunk size and non-decreasing t_kv, e.g. a
  // stream's speculative-verify rows.  Group i holds rows grp_row[i] .. + grp_n[i] - 1 and
  // runs the chunks of its longest row; the group chunk prefix sums are grp_off.
  int n_grp;
  int max_grp;
  int32_t grp_off[KD_MAX_B + 1];
  int32_t grp_row[KD_MAX_B];
  int32_t grp_n[KD_MAX_B];
  int32_t grp_chunk[KD_MAX_B];        // the rows' common chunk size
  int32_t grp_t[KD_MAX_B];            // t_kv of the group's longest (last) row
  const void* grp_k[KD_MAX_B];        // the group's K and V cache bases
  const void* grp_v[KD_MAX_B];
};
int fa_chunk_for(int t_kv);
bool fa_make_plan(FaPlan& p, int B, int H, int G, int hd, const int32_t* t_kv, int forced_chunk);
size_t fa_workspace_bytes(const FaPlan& p);
// q/out fp32 [B][H][hd] (row stride ldq / H*hd); if out_qs != nullptr the combine also
// writes the quantised output rows.
// gate (optional, row stride ldq like q): every output element is multiplied by
// sigmoid(gate) before it is written and quantised.
// kv_fmt: fp16 caches; FP8 E4M3 codes, widened to fp16 (exactly) as they are loaded; or int8
// rows (codes widened exactly, block scales applied in fp32).
void launch_fa(const FaPlan& p, const float* q, int ldq, const RowCaches& rc, int capacity, float scale,
               float* out, int8_t* out_qs, float* out_d, void* ws, hipStream_t st, const float* gate = nullptr,
               int kv_fmt = KD_KV_F16);
bool fa_shape_supported(int H, int G, int hd);
int fa_max_keys();

// Linear-attention (gated delta-rule) layers: the state step over per-row state pointers, the
// conv ring + prep, and the gated norm + quantiser of the mixer output (see gdn.hip).
int gdn_state_dim();
void launch_gdn_step(const float* q, const float* k, const float* v, const float* g, const float* beta, int B, int H,
                     const float* const* state_in, float* const* state_out, float scale, float* o, hipStream_t st);
void launch_ssm_conv_prep(const float* proj, int ldp, const float* w, int dconv, const float* const* ring_in,
                          float* const* ring_out, const float* dt, const float* a, int B, int nk, int nv, float eps,
                          float* q, float* k, float* v, float* g, float* beta, hipStream_t st);
void launch_gated_norm_quant(const float* o, const float* z, int ldz, const float* w, int B, int nv, float eps,
                             int8_t* qs, float* qd, hipStream_t st);

void launch_swiglu_quant(const float* g, const float* u, int rows, int n, int ld, float* a_out, int8_t* qs,
                         float* d, hipStream_t st);
void launch_add(const float* x, const float* y, float* z, size_t n, hipStream_t st);

// Router: logits [B][E] (written; d % 4 == 0, 16-byte aligned rows), then top-K ids and
// softmax weights per row, and per expert the (row, pair) lists routed to it (count[E],
// rows/pairs [E][16], ascending row order).
void launch_router(const float* z, const float* Wr, int B, int d, int E, int K, int32_t* ids, float* p, float* logits,
                   int32_t* count, int32_t* rows, int32_t* pairs, hipStream_t st);
int moe_max_experts();
int moe_max_topk();

}  // namespace kd
