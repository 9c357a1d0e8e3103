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

#include "kd_internal.h"

namespace kd {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kTileQ8 = 2048;
constexpr int kTileQ4 = 1024;

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
__global__ void act_quant_kernel(const float* __restrict__ x, int B, int k, int ldx, int NQ,
                                 int8_t* __restrict__ qs, float* __restrict__ d) {
  const int nb_pad = NQ * 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * nb_pad) return;
  const int b = idx / nb_pad, blk = idx % nb_pad;
  float v[32];
  if (blk * 32 < k) {
    const float4* s = reinterpret_cast<const float4*>(x + (size_t)b * ldx + blk * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 t = s[i];
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
  quant32(v, qs + ((size_t)b * NQ + (blk >> 2)) * 128 + (blk & 3) * 8, d + (size_t)b * nb_pad + blk);
}

// ---------------------------------------------------------------------------------------
// mmvq
// ---------------------------------------------------------------------------------------
__device__ inline long q4_operand(uint32_t w) {
  // Four bytes of a Q4_0 block: low nibbles = elements 4g..4g+3, high nibbles = 4g+16..4g+19.
  // Nibble n -> signed code n - 8 per byte: (n + 0x78) ^ 0x80 (no carry leaves a byte).
  uint32_t lo = w & 0x0F0F0F0Fu;
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  lo = (lo + 0x78787878u) ^ 0x80808080u;
  hi = (hi + 0x78787878u) ^ 0x80808080u;
  return (long)(((uint64_t)hi << 32) | (uint64_t)lo);
}

__device__ inline long lo64(int4 v) { return (long)(((uint64_t)(uint32_t)v.y << 32) | (uint32_t)v.x); }
__device__ inline long hi64(int4 v) { return (long)(((uint64_t)(uint32_t)v.w << 32) | (uint32_t)v.z); }

struct MmvqArgs {
  const uint8_t* wq;
  const __half* wd;
  int n_out, NQ, kblocks;
  const int8_t* xq;
  const float* xd;
  int B;
  float* y;
  int ldy;
  // grouped products (blockIdx.y = group); count == nullptr for a plain product
  const int32_t* count;
  const int32_t* act_row;
  const int32_t* out_row;
  long long w_group_tiles;
  int32_t* debug_S;  // [B][n_out][kblocks] when non-null (epilogue replaced)
};

template <int FMT>
__global__ __launch_bounds__(512) void mmvq_kernel(MmvqArgs a) {
  constexpr int TILE = FMT == KD_FMT_Q8_0 ? kTileQ8 : kTileQ4;
  const int r = blockIdx.x;  // 16-row group
  const int e = blockIdx.y;  // group (expert) for grouped products
  int nrows = a.B;
  const int32_t* act_row = nullptr;
  const int32_t* out_row = nullptr;
  if (a.count) {
    nrows = a.count[e];
    if (nrows <= 0) return;
    act_row = a.act_row + e * 16;
    out_row = a.out_row + e * 16;
  }
  const int nw = blockDim.x >> 6;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, n = lane & 15;
  const int NQ = a.NQ;
  // K-slice of this wave: a function of NQ (hence of k) only.
  const int q0 = (w * NQ) / nw, q1 = ((w + 1) * NQ) / nw;
  const int ns = nrows < 4 ? nrows : 4;  // epilogue slots that can hold a live row

  const size_t tile0 = (size_t)e * (size_t)a.w_group_tiles + (size_t)r * NQ;
  const uint8_t* wt = a.wq + tile0 * TILE + lane * 16;
  const __half* dt = a.wd + tile0 * 64 + n * 4;

  // A operand: activation row of lane's i = n
  const bool a_live = n < nrows;
  const int a_row = a_live ? (act_row ? act_row[n] : n) : 0;
  const int8_t* ap = a.xq + (size_t)a_row * NQ * 128 + g * 32;
  // epilogue rows of lane's slots: i = 4g + s
  int s_row[4];
  bool s_live[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int i = 4 * g + s;
    s_live[s] = (s < ns) && (i < nrows);
    s_row[s] = s_live[s] ? (act_row ? act_row[i] : i) : 0;
  }
  const int nbp = NQ * 4;

  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const v4i zero = {0, 0, 0, 0};

  for (int q = q0; q < q1; ++q) {
    int4 w0 = *reinterpret_cast<const int4*>(wt + (size_t)q * TILE);
    int4 w1 = w0;
    if (FMT == KD_FMT_Q8_0) w1 = *reinterpret_cast<const int4*>(wt + (size_t)q * TILE + 1024);
    const uint2 dwr = *reinterpret_cast<const uint2*>(dt + (size_t)q * 64);
    int4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
    if (a_live) {
      a0 = *reinterpret_cast<const int4*>(ap + (size_t)q * 128);
      a1 = *reinterpret_cast<const int4*>(ap + (size_t)q * 128 + 16);
    }
    float4 dx[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      dx[s] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (s < ns && s_live[s]) dx[s] = *reinterpret_cast<const float4*>(a.xd + (size_t)s_row[s] * nbp + q * 4);
    }
    float dw[4];
    dw[0] = __half2float(__ushort_as_half((unsigned short)(dwr.x & 0xFFFF)));
    dw[1] = __half2float(__ushort_as_half((unsigned short)(dwr.x >> 16)));
    dw[2] = __half2float(__ushort_as_half((unsigned short)(dwr.y & 0xFFFF)));
    dw[3] = __half2float(__ushort_as_half((unsigned short)(dwr.y >> 16)));

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long A = (j == 0) ? lo64(a0) : (j == 1) ? hi64(a0) : (j == 2) ? lo64(a1) : hi64(a1);
      long Bw;
      if (FMT == KD_FMT_Q8_0) {
        Bw = (j == 0) ? lo64(w0) : (j == 1) ? hi64(w0) : (j == 2) ? lo64(w1) : hi64(w1);
      } else {
        const uint32_t word = (j == 0) ? (uint32_t)w0.x : (j == 1) ? (uint32_t)w0.y : (j == 2) ? (uint32_t)w0.z : (uint32_t)w0.w;
        Bw = q4_operand(word);
      }
      const v4i S = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, Bw, zero, 0, 0, 0);
      if (a.debug_S) {
        const int blk = 4 * q + j;
        const int row = r * 16 + n;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int i = 4 * g + s;
          if (i < nrows && row < a.n_out && blk < a.kblocks)
            a.debug_S[((size_t)i * a.n_out + row) * a.kblocks + blk] = S[s];
        }
        continue;
      }
      const float dxs[4] = {j == 0 ? dx[0].x : j == 1 ? dx[0].y : j == 2 ? dx[0].z : dx[0].w,
                            j == 0 ? dx[1].x : j == 1 ? dx[1].y : j == 2 ? dx[1].z : dx[1].w,
                            j == 0 ? dx[2].x : j == 1 ? dx[2].y : j == 2 ? dx[2].z : dx[2].w,
                            j == 0 ? dx[3].x : j == 1 ? dx[3].y : j == 2 ? dx[3].z : dx[3].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < ns) acc[s] = fmaf(dw[j] * dxs[s], (float)S[s], acc[s]);
      }
    }
  }
  if (a.debug_S) return;

  __shared__ float red[8][4][64];
#pragma unroll
  for (int s = 0; s < 4; ++s) red[w][s][lane] = acc[s];
  __syncthreads();
  for (int t = threadIdx.x; t < 256; t += blockDim.x) {  // 256 (slot, lane) outputs, any wave count
    const int s = t >> 6, l = t & 63;
    float v = red[0][s][l];
    for (int ww = 1; ww < nw; ++ww) v += red[ww][s][l];  // fixed wave order
    const int i = 4 * (l >> 4) + s;
    const int row = r * 16 + (l & 15);
    if (i < nrows && row < a.n_out) {
      const int orow = out_row ? out_row[i] : i;
      a.y[(size_t)orow * a.ldy + row] = v;
    }
  }
}

// Waves per workgroup: a function of the quad count only (never of B).
static int mmvq_waves(int NQ) { return NQ >= 8 ? 8 : NQ; }

void launch_mmvq(const kd_weight& W, const int8_t* xq, const float* xd, int B, float* y, int ldy,
                 hipStream_t st, const RowMap* map, int32_t* debug_S) {
  MmvqArgs a;
  a.wq = static_cast<const uint8_t*>(W.qs);
  a.wd = static_cast<const __half*>(W.d);
  a.n_out = W.n_out;
  a.NQ = n_quads(W.k);
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
  a.debug_S = debug_S;
  const int NR = n_rowgroups(W.n_out);
  dim3 grid(NR, map ? map->n_groups : 1);
  dim3 block(64 * mmvq_waves(a.NQ));
  if (W.fmt == KD_FMT_Q8_0)
    mmvq_kernel<KD_FMT_Q8_0><<<grid, block, 0, st>>>(a);
  else
    mmvq_kernel<KD_FMT_Q4_0><<<grid, block, 0, st>>>(a);
}

void launch_act_quant(const float* x, int B, int k, int ldx, int8_t* qs, float* d, hipStream_t st) {
  const int NQ = n_quads(k);
  const int total = B * NQ * 4;
  act_quant_kernel<<<ceil_div(total, 256), 256, 0, st>>>(x, B, k, ldx, NQ, qs, d);
}

}  // namespace kd

using namespace kd;

// ---------------------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------------------
static bool fmt_quant(int32_t fmt) { return fmt == KD_FMT_Q8_0 || fmt == KD_FMT_Q4_0; }

extern "C" size_t kd_weight_qs_bytes(int32_t fmt, int32_t n_out, int32_t k) {
  if (!fmt_quant(fmt) || n_out <= 0 || k <= 0 || k % 32) return 0;
  const size_t tiles = (size_t)n_rowgroups(n_out) * n_quads(k);
  return tiles * (fmt == KD_FMT_Q8_0 ? kTileQ8 : kTileQ4);
}

extern "C" size_t kd_weight_d_bytes(int32_t fmt, int32_t n_out, int32_t k) {
  if (!fmt_quant(fmt) || n_out <= 0 || k <= 0 || k % 32) return 0;
  return (size_t)n_rowgroups(n_out) * n_quads(k) * 64 * sizeof(__half);
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
  KD_REQUIRE(fmt_quant(fmt), KD_ERR_UNSUPPORTED, "kd_pack_weight: format %d is not Q8_0 or Q4_0", fmt);
  KD_REQUIRE(n_out > 0 && k > 0, KD_ERR_INVALID, "kd_pack_weight: bad shape %d x %d", n_out, k);
  KD_REQUIRE(k % 32 == 0, KD_ERR_UNSUPPORTED, "kd_pack_weight: k=%d is not a multiple of 32", k);
  KD_REQUIRE(src_qs && src_d && dst_qs && dst_d, KD_ERR_INVALID, "kd_pack_weight: null pointer");
  KD_REQUIRE(aligned16(src_qs) && aligned16(dst_qs) && aligned16(dst_d), KD_ERR_INVALID,
             "kd_pack_weight: qs/d buffers must be 16-byte aligned");
  const int NR = n_rowgroups(n_out), NQ = n_quads(k);
  const long long total = (long long)NR * 16 * NQ * 4;
  const int blocks = (int)((total + 255) / 256);
  hipStream_t st = as_stream(stream);
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
  KD_REQUIRE(W->k % 32 == 0, KD_ERR_UNSUPPORTED, "%s: k=%d is not a multiple of 32", who, W->k);
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

extern "C" kd_status kd_debug_block_dots(const kd_weight* W, kd_act_q8 x, int32_t B, int32_t* S, void* stream) {
  KD_REQUIRE(W, KD_ERR_INVALID, "kd_debug_block_dots: null weight");
  kd_status s = check_mmvq_args("kd_debug_block_dots", W, W->fmt, x, B);
  if (s != KD_OK) return s;
  KD_REQUIRE(fmt_quant(W->fmt), KD_ERR_UNSUPPORTED, "kd_debug_block_dots: format %d", W->fmt);
  KD_REQUIRE(S, KD_ERR_INVALID, "kd_debug_block_dots: null output");
  launch_mmvq(*W, x.qs, x.d, B, nullptr, 0, as_stream(stream), nullptr, S);
  return check_launch("kd_debug_block_dots");
}
