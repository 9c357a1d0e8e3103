// Block-quantised matrix x B activation rows (mmvq at m = B) on MI355X, plus the weight
// repack into the MFMA tile layout and the activation quantiser that feeds it.
//
// What is computed: y[b][n] = sum_blk d_w[n][blk] * d_x[b][blk] * S[b][n][blk] with S the
// exact int32 dot product of one 32-element block of int8 codes (memra-engine 0.72.0,
// src/decode_batch.rs: ``matmul_pre`` at m = B on pre-quantised rows, one weight read
// serving all B rows; hf2q ADR-040 §0.7 F3, small-m quantised decode GEMM).
//
// How (gfx950): one v_mfma_i32_16x16x32_i8 per (16 weight rows x 1 block x 16 activation
// rows) computes 256 exact block dots at once, K = 32 = one quantisation block, so no
// integer sum ever mixes two scales.  A wave streams a contiguous range of block quads of
// one 16-row group with coalesced 16-byte loads and reuses every weight register for all B
// activation rows; the fp32 epilogue acc = fma(d_w * d_x, float(S), acc) runs per block in
// ascending block order.  The waves of a workgroup split the quads of the row group by a
// rule that depends on k only, and their partial sums are added in wave order through
// LDS.  Hence each output's fp32 operation sequence is fixed by k: row b of a B-row call
// equals the 1-row call bit for bit (memra-engine decode_batch.rs exactness contract;
// hf2q ADR-040 §0.12, dense matmul row identity).
#include <cstdio>

#include "mmvq_impl.h"

namespace kd {

// ---------------------------------------------------------------------------------------
// Weight repack: row-major blocks -> tiles (see kd.h "Native layouts").
// ---------------------------------------------------------------------------------------
template <int FMT>
__global__ void pack_weight_kernel(const uint8_t* __restrict__ src_qs, const __half* __restrict__ src_d,
                                   int n_out, int k, int NR, int NQ, uint8_t* __restrict__ dst_qs,
                                   __half* __restrict__ dst_d) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int nb_pad = NQ * 4;
  if (idx >= (long long)NR * 16 * nb_pad) return;
  const int row = (int)(idx / nb_pad), blk = (int)(idx % nb_pad);
  const int kb = k / 32;
  const bool valid = row < n_out && blk < kb;
  const int r = row >> 4, nn = row & 15, q = blk >> 2, j = blk & 3;
  const size_t t = (size_t)r * NQ + q;
  dst_d[t * 64 + nn * 4 + j] = valid ? src_d[(size_t)row * kb + blk] : __float2half(0.0f);
  if (FMT == KD_FMT_Q8_0) {
    uint32_t c[8];
    for (int i = 0; i < 8; ++i) c[i] = 0;
    if (valid) {
      const uint32_t* s = reinterpret_cast<const uint32_t*>(src_qs + (size_t)row * k + blk * 32);
      for (int i = 0; i < 8; ++i) c[i] = s[i];
    }
    // lane chunk of group g: elements 4g..4g+3 (word g) then 4g+16..4g+19 (word g+4)
    for (int g = 0; g < 4; ++g) {
      const int lane = g * 16 + nn;
      uint32_t* dst = reinterpret_cast<uint32_t*>(dst_qs + t * kTileQ8 + (j >> 1) * 1024 + lane * 16 + (j & 1) * 8);
      dst[0] = c[g];
      dst[1] = c[g + 4];
    }
  } else {
    uint32_t c[4] = {0, 0, 0, 0};
    if (valid) {
      const uint32_t* s = reinterpret_cast<const uint32_t*>(src_qs + (size_t)row * (k / 2) + blk * 16);
      for (int i = 0; i < 4; ++i) c[i] = s[i];
    }
    for (int g = 0; g < 4; ++g) {
      const int lane = g * 16 + nn;
      *reinterpret_cast<uint32_t*>(dst_qs + t * kTileQ4 + lane * 16 + j * 4) = c[g];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Activation quantiser: one thread per (row, block).
// ---------------------------------------------------------------------------------------
// grid (ceil(blocks / 32), rows); 8 lanes per 32-element block.
__global__ __launch_bounds__(256) void act_quant_kernel(const float* __restrict__ x, int k, int ldx, int NQ,
                                                        int8_t* __restrict__ qs, float* __restrict__ d) {
  const int b = blockIdx.y;
  const int sub = threadIdx.x & 7;
  const int blk = blockIdx.x * 32 + (threadIdx.x >> 3);
  const int nbp = NQ * 4;
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (blk * 32 < k) v = *reinterpret_cast<const float4*>(x + (size_t)b * ldx + blk * 32 + 4 * sub);
  quant4_lane8(v, sub, blk < nbp, qs + ((size_t)b * NQ + (blk >> 2)) * 128 + (blk & 3) * 8, d + (size_t)b * nbp + blk);
}

static MmvqArgs mmvq_args(const kd_weight& W, const int8_t* xq, const float* xd, int B, float* y, int ldy,
                          const RowMap* map, int32_t* debug_S) {
  MmvqArgs a = {};
  a.wq = static_cast<const uint8_t*>(W.qs);
  a.wd = static_cast<const __half*>(W.d);
  a.n_out = W.n_out;
  a.NR = n_rowgroups(W.n_out);
  a.NQ = n_quads(W.k);
  a.QW = mmvq_qw(a.NQ);
  a.kblocks = W.k / 32;
  a.xq = xq;
  a.xd = xd;
  a.B = B;
  a.y = y;
  a.ldy = ldy;
  a.count = map ? map->count : nullptr;
  a.act_row = map ? map->act_row : nullptr;
  a.out_row = map ? map->out_row : nullptr;
  a.w_group_tiles = map ? map->w_group_tiles : 0;
  a.n_groups = map ? map->n_groups : 1;
  a.debug_S = debug_S;
  const size_t tiles = (size_t)(map ? map->n_groups : 1) * (map ? (size_t)map->w_group_tiles : (size_t)a.NR * a.NQ);
  a.w_bytes = (uint32_t)(tiles * tile_qs_bytes(W.fmt));
  a.d_bytes = (uint32_t)(tiles * tile_d_bytes(W.fmt));
  const size_t rows = map ? (size_t)map->act_rows : (size_t)B;
  a.x_bytes = (uint32_t)(rows * a.NQ * 128);
  a.xd_bytes = (uint32_t)(rows * a.NQ * 16);
  return a;
}

template <int RG, int EPI>
static void launch_mmvq_fmt(const kd_weight& W, const MmvqArgs& a, int ng, hipStream_t st) {
  if (W.fmt == KD_FMT_Q8_0)
    launch_mmvq_t<KD_FMT_Q8_0, RG, EPI>(a, ng, st);
  else if (W.fmt == KD_FMT_Q4_0)
    launch_mmvq_t<KD_FMT_Q4_0, RG, EPI>(a, ng, st);
  else
    launch_mmvq_kq<RG, EPI>(W.fmt, a, ng, st);
}

void launch_mmvq(const kd_weight& W, const int8_t* xq, const float* xd, int B, float* y, int ldy,
                 hipStream_t st, const RowMap* map, int32_t* debug_S, const float* mo_y, const float* mo_p, int mo_K) {
  MmvqArgs a = mmvq_args(W, xq, xd, B, y, ldy, map, debug_S);
  a.mo_y = mo_y;
  a.mo_p = mo_p;
  a.mo_K = mo_K;
  // grouped Q4_0 products (the experts' down product: small k, so a workgroup of one row
  // group has little to stream) take four row groups per workgroup
  if (map && W.fmt == KD_FMT_Q4_0)
    launch_mmvq_fmt<4, EPI_PLAIN>(W, a, map->n_groups, st);
  else
    launch_mmvq_fmt<kPlainRG, EPI_PLAIN>(W, a, map ? map->n_groups : 1, st);
}

bool mmvq_swiglu_merges(const kd_weight& W, const kd_weight& X) {
  return (W.fmt == KD_FMT_Q4_0 || W.fmt == KD_FMT_Q8_0) && X.fmt == W.fmt && X.k == W.k && W.n_out % 64 == 0 &&
         X.n_out % W.n_out == 0 && X.n_out / W.n_out <= 8 && X.qs && X.d;
}

void launch_mmvq_swiglu(const kd_weight& W, const int8_t* xq, const float* xd, int B, int8_t* out_qs, float* out_d,
                        hipStream_t st, const float* norm_ss, int norm_n, float norm_eps, const RowMap* map,
                        const kd_weight* X, int8_t* x_qs, float* x_qd) {
  MmvqArgs a = mmvq_args(W, xq, xd, B, nullptr, 0, map, nullptr);
  if (map && X) {  // the extra matrix's slices as groups after the row map's
    a.x_groups = X->n_out / W.n_out;
    a.x_wq = static_cast<const uint8_t*>(X->qs);
    a.x_wd = static_cast<const __half*>(X->d);
    const size_t xt = (size_t)n_rowgroups(X->n_out) * a.NQ;
    a.x_w_bytes = (uint32_t)(xt * tile_qs_bytes(X->fmt));
    a.x_d_bytes = (uint32_t)(xt * tile_d_bytes(X->fmt));
    a.x_qs = x_qs;
    a.x_qd = x_qd;
  }
  a.epi_qs = out_qs;
  a.epi_qd = out_d;
  a.norm_ss = norm_ss;
  a.norm_n = norm_n;
  a.norm_eps = norm_eps;
  a.QW = mmvq_qw(a.NQ, kQuadsSW);
  launch_mmvq_fmt<4, EPI_SWIGLU>(W, a, map ? map->n_groups + a.x_groups : 1, st);
}

// Two row groups per workgroup (one 32-element block of the residual row); two quads per
// wave, so the workgroup count halves but the wave count does not.  Two or more rows are
// split over two grid slices (each workgroup streams its 32 weight rows for half the rows;
// above four rows, with half the epilogue slots per tile), so the launch fills twice the
// CUs.  The two slices
// of a block are gridDim.x workgroups apart in dispatch order: on one XCD, and its L2, when
// gridDim.x is a multiple of 8.
void launch_mmvq_resnorm(const kd_weight& W, const int8_t* xq, const float* xd, int B, const float* res, int ld,
                         const float* gain, float* x1, int8_t* out_qs, float* out_d, float* ss, hipStream_t st) {
  MmvqArgs a = mmvq_args(W, xq, xd, B, nullptr, 0, nullptr, nullptr);
  a.QW = mmvq_qw(a.NQ, kQuadsRN);
  if (B > 4)
    a.row_split = 4 * ceil_div(ceil_div(B, 4), 2);
  else if (B > 1)
    a.row_split = ceil_div(B, 2);
  a.epi_res = res;
  a.epi_ld = ld;
  a.epi_gain = gain;
  a.epi_x1 = x1;
  a.epi_qs = out_qs;
  a.epi_qd = out_d;
  a.epi_ss = ss;
  launch_mmvq_fmt<2, EPI_RESNORM>(W, a, 1, st);
}

void launch_mmvq_rope(const kd_weight& W, const int8_t* xq, const float* xd, int B, float* q, int ldq, int H, int G,
                      int hd, const float* cs, float rope_base, const RowCaches& rc, int capacity, hipStream_t st,
                      const float* norm_ss, int norm_n, float norm_eps, bool kv_fp8) {
  MmvqArgs a = mmvq_args(W, xq, xd, B, nullptr, 0, nullptr, nullptr);
  a.norm_ss = norm_ss;
  a.norm_n = norm_n;
  a.norm_eps = norm_eps;
  a.epi_kv8 = kv_fp8 ? 1 : 0;
  a.epi_base = (double)rope_base;
  a.epi_q = q;
  a.epi_ldq = ldq;
  a.epi_H = H;
  a.epi_G = G;
  a.epi_hd = hd;
  a.epi_cs = cs;
  a.epi_rc = rc;
  a.epi_capacity = capacity;
  a.QW = mmvq_qw(a.NQ, kQuadsRope);
  launch_mmvq_fmt<1, EPI_ROPE>(W, a, 1, st);
}

// A product's limits: k up to kMaxK (the widest wave partition), and the tiled codes and
// scales addressable by 32-bit buffer offsets with kOOB past their end.
bool mmvq_weight_fits(int fmt, int n_out, int k) {
  if (n_out <= 0 || k <= 0 || k > kMaxK) return false;
  const size_t tiles = (size_t)n_rowgroups(n_out) * n_quads(k);
  const size_t qs = tiles * tile_qs_bytes(fmt);
  return qs < (size_t)kOOB && tiles * tile_d_bytes(fmt) < (size_t)kOOB;
}
int mmvq_max_k() { return kMaxK; }

// The quantised weight formats, and the column multiple each needs (one block / record).
bool mmvq_fmt_ok(int fmt, int k) {
  if (fmt == KD_FMT_Q8_0 || fmt == KD_FMT_Q4_0) return k > 0 && k % 32 == 0;
  return fmt_is_kq(fmt) && k > 0 && k % 256 == 0;
}

// LDS of the SwiGLU product (four row groups per workgroup: the largest of the products),
// which bounds its k below kMaxK on a 160 KiB-LDS CU.
static size_t swiglu_lds_bytes(int k) {
  const int NQ = n_quads(k), QW = mmvq_qw(NQ, kQuadsSW), nw = ceil_div(NQ, QW);
  return (size_t)nw * mmvq_wave_lds(QW, 4) + (size_t)nw * 4 * 256 * sizeof(float) + 4 * 256 * sizeof(float);
}
bool mmvq_swiglu_fits(int k) { return swiglu_lds_bytes(k) <= 160u * 1024u; }

void launch_act_quant(const float* x, int B, int k, int ldx, int8_t* qs, float* d, hipStream_t st) {
  const int NQ = n_quads(k);
  act_quant_kernel<<<dim3(ceil_div(NQ * 4, 32), B), 256, 0, st>>>(x, k, ldx, NQ, qs, d);
}

}  // namespace kd

using namespace kd;

// ---------------------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------------------
static bool fmt_quant(int32_t fmt) { return fmt == KD_FMT_Q8_0 || fmt == KD_FMT_Q4_0 || fmt_is_kq(fmt); }

extern "C" size_t kd_weight_qs_bytes(int32_t fmt, int32_t n_out, int32_t k) {
  if (!mmvq_fmt_ok(fmt, k) || n_out <= 0) return 0;
  const size_t tiles = (size_t)n_rowgroups(n_out) * n_quads(k);
  return tiles * tile_qs_bytes(fmt);
}

extern "C" size_t kd_weight_d_bytes(int32_t fmt, int32_t n_out, int32_t k) {
  if (!mmvq_fmt_ok(fmt, k) || n_out <= 0) return 0;
  return (size_t)n_rowgroups(n_out) * n_quads(k) * tile_d_bytes(fmt);
}

extern "C" size_t kd_act_qs_bytes(int32_t B, int32_t k) {
  if (B <= 0 || k <= 0 || k % 32) return 0;
  return (size_t)B * n_quads(k) * 128;
}

extern "C" size_t kd_act_d_bytes(int32_t B, int32_t k) {
  if (B <= 0 || k <= 0 || k % 32) return 0;
  return (size_t)B * n_quads(k) * 4 * sizeof(float);
}

extern "C" kd_status kd_pack_weight(int32_t fmt, int32_t n_out, int32_t k, const void* src_qs, const void* src_d,
                                    void* dst_qs, void* dst_d, void* stream) {
  KD_REQUIRE(fmt_quant(fmt), KD_ERR_UNSUPPORTED, "kd_pack_weight: format %d is not a quantised weight format", fmt);
  KD_REQUIRE(n_out > 0 && k > 0, KD_ERR_INVALID, "kd_pack_weight: bad shape %d x %d", n_out, k);
  KD_REQUIRE(mmvq_fmt_ok(fmt, k), KD_ERR_UNSUPPORTED, "kd_pack_weight: k=%d is not a multiple of %d", k,
             fmt_is_kq(fmt) ? 256 : 32);
  KD_REQUIRE(kd_weight_qs_bytes(fmt, n_out, k) < (size_t)kOOB, KD_ERR_UNSUPPORTED,
             "kd_pack_weight: %d x %d: tiled codes reach 2 GiB", n_out, k);
  hipStream_t st = as_stream(stream);
  if (fmt_is_kq(fmt)) {  // records carry their scales: src_d unused
    KD_REQUIRE(src_qs && dst_qs && dst_d, KD_ERR_INVALID, "kd_pack_weight: null pointer");
    KD_REQUIRE(aligned16(dst_qs) && aligned16(dst_d), KD_ERR_INVALID, "kd_pack_weight: dst buffers must be 16-byte aligned");
    launch_pack_kquant(fmt, static_cast<const uint8_t*>(src_qs), n_out, k, static_cast<uint8_t*>(dst_qs),
                       static_cast<uint8_t*>(dst_d), st);
    return check_launch("kd_pack_weight");
  }
  KD_REQUIRE(src_qs && src_d && dst_qs && dst_d, KD_ERR_INVALID, "kd_pack_weight: null pointer");
  KD_REQUIRE(aligned16(src_qs) && aligned16(dst_qs) && aligned16(dst_d), KD_ERR_INVALID,
             "kd_pack_weight: qs/d buffers must be 16-byte aligned");
  const int NR = n_rowgroups(n_out), NQ = n_quads(k);
  const long long total = (long long)NR * 16 * NQ * 4;
  const int blocks = (int)((total + 255) / 256);
  if (fmt == KD_FMT_Q8_0)
    pack_weight_kernel<KD_FMT_Q8_0><<<blocks, 256, 0, st>>>(static_cast<const uint8_t*>(src_qs),
                                                            static_cast<const __half*>(src_d), n_out, k, NR, NQ,
                                                            static_cast<uint8_t*>(dst_qs), static_cast<__half*>(dst_d));
  else
    pack_weight_kernel<KD_FMT_Q4_0><<<blocks, 256, 0, st>>>(static_cast<const uint8_t*>(src_qs),
                                                            static_cast<const __half*>(src_d), n_out, k, NR, NQ,
                                                            static_cast<uint8_t*>(dst_qs), static_cast<__half*>(dst_d));
  return check_launch("kd_pack_weight");
}

extern "C" kd_status kd_quantize_act_q8(const float* x, int32_t B, int32_t k, int32_t ldx, kd_act_q8 out,
                                        void* stream) {
  KD_REQUIRE(B >= 1 && B <= KD_MAX_B, KD_ERR_UNSUPPORTED, "kd_quantize_act_q8: B=%d outside [1,16]", B);
  KD_REQUIRE(k > 0 && k % 32 == 0, KD_ERR_UNSUPPORTED, "kd_quantize_act_q8: k=%d is not a positive multiple of 32", k);
  KD_REQUIRE(ldx >= k && ldx % 4 == 0, KD_ERR_INVALID, "kd_quantize_act_q8: ldx=%d must be >= k and a multiple of 4", ldx);
  KD_REQUIRE(x && out.qs && out.d, KD_ERR_INVALID, "kd_quantize_act_q8: null pointer");
  KD_REQUIRE(aligned16(x) && aligned16(out.qs) && aligned16(out.d), KD_ERR_INVALID,
             "kd_quantize_act_q8: buffers must be 16-byte aligned");
  launch_act_quant(x, B, k, ldx, out.qs, out.d, as_stream(stream));
  return check_launch("kd_quantize_act_q8");
}

static kd_status check_mmvq_args(const char* who, const kd_weight* W, int32_t want_fmt, kd_act_q8 x, int32_t B) {
  KD_REQUIRE(W, KD_ERR_INVALID, "%s: null weight", who);
  KD_REQUIRE(W->fmt == want_fmt, KD_ERR_UNSUPPORTED, "%s: weight format %d does not match this entry point", who, W->fmt);
  KD_REQUIRE(B >= 1 && B <= KD_MAX_B, KD_ERR_UNSUPPORTED, "%s: B=%d outside [1,16]", who, B);
  KD_REQUIRE(W->n_out > 0 && W->k > 0, KD_ERR_INVALID, "%s: bad shape %d x %d", who, W->n_out, W->k);
  KD_REQUIRE(mmvq_fmt_ok(W->fmt, W->k), KD_ERR_UNSUPPORTED, "%s: format %d with k=%d (k %% 32, K-quants k %% 256)", who,
             W->fmt, W->k);
  KD_REQUIRE(mmvq_weight_fits(W->fmt, W->n_out, W->k), KD_ERR_UNSUPPORTED,
             "%s: %d x %d exceeds the product's limits (k <= %d, tiled codes under 2 GiB)", who, W->n_out, W->k,
             kMaxK);
  KD_REQUIRE(W->qs && W->d && x.qs && x.d, KD_ERR_INVALID, "%s: null pointer", who);
  KD_REQUIRE(aligned16(W->qs) && aligned16(W->d) && aligned16(x.qs) && aligned16(x.d), KD_ERR_INVALID,
             "%s: buffers must be 16-byte aligned", who);
  return KD_OK;
}

static kd_status mmvq_entry(const char* who, int32_t fmt, const kd_weight* W, kd_act_q8 x, int32_t B, float* y,
                            int32_t ldy, void* stream) {
  kd_status s = check_mmvq_args(who, W, fmt, x, B);
  if (s != KD_OK) return s;
  KD_REQUIRE(y, KD_ERR_INVALID, "%s: null output", who);
  KD_REQUIRE(ldy >= W->n_out, KD_ERR_INVALID, "%s: ldy=%d < n_out=%d", who, ldy, W->n_out);
  launch_mmvq(*W, x.qs, x.d, B, y, ldy, as_stream(stream));
  return check_launch(who);
}

extern "C" kd_status kd_mmvq_q8_0(const kd_weight* W, kd_act_q8 x, int32_t B, float* y, int32_t ldy, void* stream) {
  return mmvq_entry("kd_mmvq_q8_0", KD_FMT_Q8_0, W, x, B, y, ldy, stream);
}

extern "C" kd_status kd_mmvq_q4_0(const kd_weight* W, kd_act_q8 x, int32_t B, float* y, int32_t ldy, void* stream) {
  return mmvq_entry("kd_mmvq_q4_0", KD_FMT_Q4_0, W, x, B, y, ldy, stream);
}

extern "C" kd_status kd_mmvq(const kd_weight* W, kd_act_q8 x, int32_t B, float* y, int32_t ldy, void* stream) {
  KD_REQUIRE(W, KD_ERR_INVALID, "kd_mmvq: null weight");
  KD_REQUIRE(fmt_quant(W->fmt), KD_ERR_UNSUPPORTED, "kd_mmvq: format %d is not a quantised weight format", W->fmt);
  return mmvq_entry("kd_mmvq", W->fmt, W, x, B, y, ldy, stream);
}

extern "C" kd_status kd_mmvq_swiglu(const kd_weight* W, kd_act_q8 x, int32_t B, kd_act_q8 out, void* stream) {
  const char* who = "kd_mmvq_swiglu";
  KD_REQUIRE(W, KD_ERR_INVALID, "%s: null weight", who);
  kd_status s = check_mmvq_args(who, W, W->fmt, x, B);
  if (s != KD_OK) return s;
  KD_REQUIRE(fmt_quant(W->fmt), KD_ERR_UNSUPPORTED, "%s: format %d", who, W->fmt);
  KD_REQUIRE(W->n_out % 64 == 0, KD_ERR_UNSUPPORTED, "%s: n_out=%d is not 2F with F a multiple of 32", who,
             W->n_out);
  KD_REQUIRE(mmvq_swiglu_fits(W->k), KD_ERR_UNSUPPORTED, "%s: k=%d exceeds the SwiGLU product's LDS", who, W->k);
  KD_REQUIRE(out.qs && out.d && aligned16(out.qs) && aligned16(out.d), KD_ERR_INVALID,
             "%s: output buffers null or not 16-byte aligned", who);
  launch_mmvq_swiglu(*W, x.qs, x.d, B, out.qs, out.d, as_stream(stream));
  return check_launch(who);
}

static kd_status rope_entry(const char* who, const kd_weight* W, kd_act_q8 x, int32_t B, int32_t H, int32_t G,
                            int32_t hd, float* q_out, int32_t ldq, void* const* k_base, void* const* v_base,
                            const int32_t* pos, int32_t capacity, float rope_base, const float* norm_ss, float eps,
                            void* stream) {
  KD_REQUIRE(W, KD_ERR_INVALID, "%s: null weight", who);
  kd_status s = check_mmvq_args(who, W, W->fmt, x, B);
  if (s != KD_OK) return s;
  KD_REQUIRE(fmt_quant(W->fmt), KD_ERR_UNSUPPORTED, "%s: format %d", who, W->fmt);
  KD_REQUIRE(H > 0 && G > 0 && H % G == 0, KD_ERR_INVALID, "%s: H=%d G=%d", who, H, G);
  KD_REQUIRE(hd == 64 || hd == 128, KD_ERR_UNSUPPORTED, "%s: hd=%d not 64 or 128", who, hd);
  KD_REQUIRE(W->n_out == (H + 2 * G) * hd, KD_ERR_INVALID, "%s: n_out=%d is not (H + 2G) hd = %d", who, W->n_out,
             (H + 2 * G) * hd);
  KD_REQUIRE(q_out && ldq >= H * hd, KD_ERR_INVALID, "%s: q_out null or ldq=%d < H hd", who, ldq);
  KD_REQUIRE(k_base && v_base && pos, KD_ERR_INVALID, "%s: null cache table", who);
  RowCaches rc = {};
  for (int b = 0; b < B; ++b) {
    KD_REQUIRE(k_base[b] && v_base[b], KD_ERR_INVALID, "%s: null cache pointer for row %d", who, b);
    KD_REQUIRE(pos[b] >= 0 && pos[b] + 1 <= capacity, KD_ERR_CAPACITY, "%s: pos[%d]=%d does not fit capacity %d", who,
               b, pos[b], capacity);
    for (int a = 0; a < b; ++a)
      KD_REQUIRE(!(k_base[a] == k_base[b] && pos[a] == pos[b]), KD_ERR_INVALID,
                 "%s: rows %d and %d write the same cache slot", who, a, b);
    rc.k[b] = k_base[b];
    rc.v[b] = v_base[b];
    rc.pos[b] = pos[b];
  }
  launch_mmvq_rope(*W, x.qs, x.d, B, q_out, ldq, H, G, hd, nullptr, rope_base, rc, capacity, as_stream(stream), norm_ss,
                   W->k, eps);
  return check_launch(who);
}

extern "C" kd_status kd_mmvq_rope(const kd_weight* W, kd_act_q8 x, int32_t B, int32_t H, int32_t G, int32_t hd,
                                  float* q_out, int32_t ldq, void* const* k_base, void* const* v_base,
                                  const int32_t* pos, int32_t capacity, float rope_base, void* stream) {
  return rope_entry("kd_mmvq_rope", W, x, B, H, G, hd, q_out, ldq, k_base, v_base, pos, capacity, rope_base, nullptr,
                    0.0f, stream);
}

static kd_status check_norm_ss(const char* who, const kd_weight* W, const float* norm_ss, float eps) {
  if (!norm_ss) return KD_OK;
  KD_REQUIRE(W->k <= kNormFuseMax, KD_ERR_UNSUPPORTED, "%s: a normalised input row of k=%d exceeds %d", who, W->k,
             kNormFuseMax);
  KD_REQUIRE(eps > 0.0f && aligned16(norm_ss), KD_ERR_INVALID, "%s: eps must be positive and norm_ss 16-byte aligned",
             who);
  return KD_OK;
}

extern "C" kd_status kd_mmvq_resnorm(const kd_weight* W, kd_act_q8 x, int32_t B, const float* res, const float* gain,
                                     float* x1, kd_act_q8 out, float* ss, void* stream) {
  const char* who = "kd_mmvq_resnorm";
  KD_REQUIRE(W, KD_ERR_INVALID, "%s: null weight", who);
  kd_status s = check_mmvq_args(who, W, W->fmt, x, B);
  if (s != KD_OK) return s;
  KD_REQUIRE(fmt_quant(W->fmt), KD_ERR_UNSUPPORTED, "%s: format %d", who, W->fmt);
  KD_REQUIRE(W->n_out % 32 == 0 && W->n_out <= kNormFuseMax, KD_ERR_UNSUPPORTED,
             "%s: n_out=%d must be a multiple of 32 and at most %d", who, W->n_out, kNormFuseMax);
  KD_REQUIRE(res && gain && x1 && ss && out.qs && out.d, KD_ERR_INVALID, "%s: null pointer", who);
  KD_REQUIRE(aligned16(res) && aligned16(gain) && aligned16(x1) && aligned16(out.qs) && aligned16(out.d),
             KD_ERR_INVALID, "%s: res, gain, x1 and out must be 16-byte aligned", who);
  KD_REQUIRE(res != x1, KD_ERR_INVALID, "%s: x1 may not alias res", who);
  launch_mmvq_resnorm(*W, x.qs, x.d, B, res, W->n_out, gain, x1, out.qs, out.d, ss, as_stream(stream));
  return check_launch(who);
}

extern "C" kd_status kd_mmvq_swiglu_normed(const kd_weight* W, kd_act_q8 x, int32_t B, const float* norm_ss,
                                           float eps, kd_act_q8 out, void* stream) {
  const char* who = "kd_mmvq_swiglu_normed";
  KD_REQUIRE(norm_ss, KD_ERR_INVALID, "%s: null norm_ss", who);
  KD_REQUIRE(W, KD_ERR_INVALID, "%s: null weight", who);
  kd_status s = check_norm_ss(who, W, norm_ss, eps);
  if (s != KD_OK) return s;
  s = check_mmvq_args(who, W, W->fmt, x, B);
  if (s != KD_OK) return s;
  KD_REQUIRE(fmt_quant(W->fmt), KD_ERR_UNSUPPORTED, "%s: format %d", who, W->fmt);
  KD_REQUIRE(W->n_out % 64 == 0, KD_ERR_UNSUPPORTED, "%s: n_out=%d is not 2F with F a multiple of 32", who,
             W->n_out);
  KD_REQUIRE(mmvq_swiglu_fits(W->k), KD_ERR_UNSUPPORTED, "%s: k=%d exceeds the SwiGLU product's LDS", who, W->k);
  KD_REQUIRE(out.qs && out.d && aligned16(out.qs) && aligned16(out.d), KD_ERR_INVALID,
             "%s: output buffers null or not 16-byte aligned", who);
  launch_mmvq_swiglu(*W, x.qs, x.d, B, out.qs, out.d, as_stream(stream), norm_ss, W->k, eps);
  return check_launch(who);
}

extern "C" kd_status kd_mmvq_rope_normed(const kd_weight* W, kd_act_q8 x, int32_t B, const float* norm_ss, float eps,
                                         int32_t H, int32_t G, int32_t hd, float* q_out, int32_t ldq,
                                         void* const* k_base, void* const* v_base, const int32_t* pos,
                                         int32_t capacity, float rope_base, void* stream) {
  const char* who = "kd_mmvq_rope_normed";
  KD_REQUIRE(norm_ss, KD_ERR_INVALID, "%s: null norm_ss", who);
  KD_REQUIRE(W, KD_ERR_INVALID, "%s: null weight", who);
  kd_status s = check_norm_ss(who, W, norm_ss, eps);
  if (s != KD_OK) return s;
  return rope_entry(who, W, x, B, H, G, hd, q_out, ldq, k_base, v_base, pos, capacity, rope_base, norm_ss, eps,
                    stream);
}

extern "C" kd_status kd_debug_block_dots(const kd_weight* W, kd_act_q8 x, int32_t B, int32_t* S, void* stream) {
  KD_REQUIRE(W, KD_ERR_INVALID, "kd_debug_block_dots: null weight");
  kd_status s = check_mmvq_args("kd_debug_block_dots", W, W->fmt, x, B);
  if (s != KD_OK) return s;
  KD_REQUIRE(W->fmt == KD_FMT_Q8_0 || W->fmt == KD_FMT_Q4_0, KD_ERR_UNSUPPORTED, "kd_debug_block_dots: format %d",
             W->fmt);
  KD_REQUIRE(S, KD_ERR_INVALID, "kd_debug_block_dots: null output");
  launch_mmvq(*W, x.qs, x.d, B, nullptr, 0, as_stream(stream), nullptr, S);
  return check_launch("kd_debug_block_dots");
}

extern "C" kd_status kd_debug_mmvq_grouped(const kd_weight* W, int32_t n_groups, kd_act_q8 x, int32_t act_rows,
                                           const int32_t* count, const int32_t* act_row, const int32_t* out_row,
                                           int32_t swiglu, float* y, int32_t ldy, kd_act_q8 out, void* stream) {
  const char* who = "kd_debug_mmvq_grouped";
  KD_REQUIRE(W, KD_ERR_INVALID, "%s: null weight", who);
  kd_status s = check_mmvq_args(who, W, W->fmt, x, 1);
  if (s != KD_OK) return s;
  KD_REQUIRE(fmt_quant(W->fmt), KD_ERR_UNSUPPORTED, "%s: format %d", who, W->fmt);
  KD_REQUIRE(n_groups >= 1 && W->n_out % 16 == 0, KD_ERR_UNSUPPORTED,
             "%s: n_groups=%d, rows per group %d (a multiple of 16)", who, n_groups, W->n_out);
  KD_REQUIRE(mmvq_weight_fits(W->fmt, W->n_out * n_groups, W->k), KD_ERR_UNSUPPORTED, "%s: stacked matrix too large",
             who);
  KD_REQUIRE(act_rows >= 1 && act_rows <= KD_MAX_B * 16, KD_ERR_UNSUPPORTED, "%s: act_rows=%d", who, act_rows);
  KD_REQUIRE(count && act_row && out_row, KD_ERR_INVALID, "%s: null row map", who);
  RowMap map{count, act_row, out_row, n_groups, (long long)n_rowgroups(W->n_out) * n_quads(W->k), act_rows};
  if (swiglu) {
    KD_REQUIRE(W->n_out % 64 == 0, KD_ERR_UNSUPPORTED, "%s: SwiGLU rows per group %d is not 2F, F %% 32 == 0", who,
               W->n_out);
    KD_REQUIRE(mmvq_swiglu_fits(W->k), KD_ERR_UNSUPPORTED, "%s: k=%d exceeds the SwiGLU product's LDS", who, W->k);
    KD_REQUIRE(out.qs && out.d && aligned16(out.qs) && aligned16(out.d), KD_ERR_INVALID,
               "%s: output buffers null or not 16-byte aligned", who);
    launch_mmvq_swiglu(*W, x.qs, x.d, 0, out.qs, out.d, as_stream(stream), nullptr, 0, 0.0f, &map);
  } else {
    KD_REQUIRE(y && ldy >= W->n_out, KD_ERR_INVALID, "%s: null output or ldy=%d < rows per group", who, ldy);
    launch_mmvq(*W, x.qs, x.d, 0, y, ldy, as_stream(stream), &map);
  }
  return check_launch(who);
}
