// The block-quantised mmvq kernel template and its launch dispatch, shared by the
// translation units that instantiate it (mmvq.hip: Q8_0 and Q4_0; mmvq_kq.hip: the K-quant
// formats).  What it computes and how: see mmvq.hip.
#pragma once

#include "kd_internal.h"

namespace kd {

// Launch shape constants (measured on MI355X; see the mmvq design notes).
constexpr bool kWeightNT = true;  // weight tiles are streamed once: non-temporal loads
constexpr int kDepthQ4 = 2;       // weight-ring depth, one row group per workgroup, Q4_0
constexpr int kDepthQ8 = 2;       // the same for Q8_0
constexpr int kDepthRG = 4;       // ring depth when a workgroup streams several row groups
constexpr int kDepthRN = 4;       // ring depth of the add + RMSNorm products (two row groups)
constexpr int kWaveQuads = 8;     // quads per wave of the plain product (at most: see mmvq_qw)
constexpr int kQuadsSW = 8;       // the same for the SwiGLU product
constexpr int kQuadsRope = 8;     // the same for the RoPE product
constexpr int kQuadsRN = 2;       // quads per wave of the add + RMSNorm products
constexpr int kPlainRG = 1;       // row groups per workgroup of the plain product
// the largest k a product takes: 16 waves of kWaveQuads quads of 128 elements
constexpr int kMaxK = 16 * kWaveQuads * 128;

constexpr int kTileQ8 = 2048;
constexpr int kTileQ4 = 1024;

// Tile bytes of each weight format (16 rows x one quad of 128 columns; see kd.h "Native
// layouts"): codes, and scales.  The K-quant tiles hold the 4-bit codes as Q4_0 does, then
// the fifth bits (Q5_K, 1 byte per lane and block) or the upper two bits (Q6_K, 2 bytes per
// lane and block); their scale tiles hold, per column, the quad's four sub-block scale/min
// byte pairs (Q6_K: the two int8 scales of each 32-value block) and the super-block's fp16
// d and dmin.
__host__ __device__ constexpr bool fmt_is_kq(int fmt) {
  return fmt == KD_FMT_Q4_K || fmt == KD_FMT_Q5_K || fmt == KD_FMT_Q6_K;
}
__host__ __device__ constexpr int tile_qs_bytes(int fmt) {
  return fmt == KD_FMT_Q8_0 ? kTileQ8 : fmt == KD_FMT_Q5_K ? 1280 : fmt == KD_FMT_Q6_K ? 1536 : kTileQ4;
}
__host__ __device__ constexpr int tile_d_bytes(int fmt) { return fmt_is_kq(fmt) ? 192 : 128; }

// ---------------------------------------------------------------------------------------
// mmvq
// ---------------------------------------------------------------------------------------
__device__ inline long lo64(int4 v) { return (long)(((uint64_t)(uint32_t)v.y << 32) | (uint32_t)v.x); }
__device__ inline long hi64(int4 v) { return (long)(((uint64_t)(uint32_t)v.w << 32) | (uint32_t)v.z); }

struct MmvqArgs {
  const uint8_t* wq;
  const __half* wd;
  uint32_t w_bytes, d_bytes, x_bytes, xd_bytes;  // buffer extents (reads past them return 0)
  int n_out, NR, NQ, QW, kblocks;
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
  // fused epilogues (plain products leave these unused)
  int8_t* epi_qs;     // SwiGLU: quantised silu(gate) * up rows, F = n_out / 2 columns
  float* epi_qd;
  float* epi_q;       // RoPE: rotated q rows (stride epi_ldq); k and v go to the caches
  const float* epi_cs;  // cos/sin table [B][hd/2][2], or null: evaluated here from epi_base
  double epi_base;
  int epi_ldq, epi_H, epi_G, epi_hd, epi_capacity;
  RowCaches epi_rc;
  // add + RMSNorm: x1 = res + y (stride epi_ld), x1 * gain quantised into epi_qs/epi_qd, and
  // per (row, 32-element block) sums of x1^2 into epi_ss [B][n_out / 32]
  const float* epi_res;
  float* epi_x1;
  const float* epi_gain;
  float* epi_ss;
  int epi_ld;
  // normalised input (SwiGLU): every output of row b is scaled by
  // 1 / sqrt(sum_blk norm_ss[b][blk] / norm_n + norm_eps); null: no scaling
  const float* norm_ss;
  int norm_n;
  float norm_eps;
  int epi_kv8;  // RoPE: the caches hold FP8 E4M3 codes (else fp16)
  // add + RMSNorm launches: activation rows per grid z slice (slice z takes rows
  // [z row_split, min(B, (z + 1) row_split))); 0: one slice of all B rows
  int row_split;
  // grouped SwiGLU launches: n_groups groups from the row map, then x_groups more that cut an
  // extra matrix (x_wq / x_wd: the shared expert's, x_groups times a group's rows) into
  // slices of w_group_tiles tiles and apply each to all B rows; slice c writes output columns
  // [c F, (c + 1) F) of the x_qs / x_qd rows (F = n_out / 2 per slice)
  int n_groups, x_groups;
  const uint8_t* x_wq;
  const __half* x_wd;
  uint32_t x_w_bytes, x_d_bytes;
  int8_t* x_qs;
  float* x_qd;
  // plain product writing a MoE layer's output (mo_y != nullptr): y[b][row] = sum_k
  // mo_p[b][k] mo_y[b K + k][row] (rank order, fma from 0) + (W x)[b][row] -- the experts' rows
  // and this product (the shared expert's down), as the separate combine adds them
  const float* mo_y;
  const float* mo_p;
  int mo_K;
};

// Epilogue of a product: write y (plain); apply SwiGLU to the interleaved gate/up rows and
// quantise the result (swiglu); rotate q/k pairs and store q, and k and v in the caches (rope);
// add the residual, quantise x1 * gain and record the sums of squares of x1 (resnorm).
enum { EPI_PLAIN = 0, EPI_SWIGLU = 1, EPI_ROPE = 2, EPI_RESNORM = 3 };

// RMSNorm split across two products.  The producer (resnorm epilogue, 32 output rows per
// workgroup = one block) quantises z = x1 * gain with the block's own scale and writes the
// block's sum of squares of x1.  The consumer scales each output of row b by
// inv_b = 1 / sqrt(sum of the row's block sums / n + eps): the block scale max|z|/127 times
// inv_b is the scale of the normalised block y = x1 * inv_b * gain, and the codes of z and y
// are the same numbers.  The row's blocks are added by its 8 lanes: lane `sub` adds blocks
// [sub * c, sub * c + c) in order (c = ceil(blocks / 8) <= kNormPerLane), then the 8 lanes by
// DPP sum over the 8-lane group (group8_sum: every lane ends with the same value).  A lane
// fetches its sums in 16-byte loads when they come in whole quads (c a multiple of 4 and 8c
// blocks per row), else one by one; the sums and their order are the same.
constexpr int kNormPerLane = 16;  // block sums per lane: rows of up to 8 * 16 * 32 = 4096

__device__ __forceinline__ void norm_ss_load(const MmvqArgs& a, int t, int nrows, float (&v)[kNormPerLane]) {
  const int bq = t >> 3, sub = t & 7;
  const int nblk = a.norm_n / 32, c = (nblk + 7) / 8;
  // no sums (plain SwiGLU): an empty range, every load reads zero without touching memory
  const __amdgpu_buffer_rsrc_t r =
      a.norm_ss ? make_rsrc(a.norm_ss, (uint32_t)(nrows * nblk * 4)) : make_rsrc(a.xd, 0u);
  if (nblk == 8 * c && (c & 3) == 0) {  // whole 16-byte quads of sums: c / 4 wide loads
#pragma unroll
    for (int i4 = 0; i4 < kNormPerLane / 4; ++i4) {
      const int blk = sub * c + 4 * i4;
      const int4 q4 = buf16<0>(r, (bq < nrows && 4 * i4 < c) ? (uint32_t)(bq * nblk + blk) * 4u : kOOB);
      v[4 * i4] = __int_as_float(q4.x);
      v[4 * i4 + 1] = __int_as_float(q4.y);
      v[4 * i4 + 2] = __int_as_float(q4.z);
      v[4 * i4 + 3] = __int_as_float(q4.w);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kNormPerLane; ++i) {
    const int blk = sub * c + i;
    v[i] = buf4f(r, (bq < nrows && i < c && blk < nblk) ? (uint32_t)(bq * nblk + blk) * 4u : kOOB);
  }
}

__device__ __forceinline__ float norm_inv(const MmvqArgs& a, const float (&v)[kNormPerLane]) {
  float s = v[0];
#pragma unroll
  for (int i = 1; i < kNormPerLane; ++i) s += v[i];
  s = group8_sum(s);
  return 1.0f / sqrtf(s / (float)a.norm_n + a.norm_eps);
}

// Sum over the waves of the workgroup, in wave order, of output (r, s, l) of the partials
// red[wave][r][s][64]: every read is issued before the adds (nw <= 16).
template <int RG>
__device__ __forceinline__ float sum_waves(const float* red, int nw, int r, int s, int l) {
  float v = red[(r * 4 + s) * 64 + l];
  float x[15];
#pragma unroll
  for (int ww = 1; ww < 16; ++ww) x[ww - 1] = ww < nw ? red[((ww * RG + r) * 4 + s) * 64 + l] : 0.0f;
#pragma unroll
  for (int ww = 1; ww < 16; ++ww)
    if (ww < nw) v += x[ww - 1];
  return v;
}

// Batch rows on the MFMA operand: operand row i (accumulator slot s = i % 4 of lane group
// i / 4) holds activation row (i / 4) + 4 (i % 4), so B rows fill slots 0 .. ceil(B/4) - 1 of
// every lane group and the fp32 epilogue runs ceil(B/4) slots instead of min(B, 4).
__device__ __forceinline__ int mfma_row_b(int i) { return (i >> 2) + 4 * (i & 3); }

__device__ __forceinline__ float f4_get(const float4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// The A operand of lane n for the 4 blocks of one quad: 32 bytes (2 x 16-byte loads).
__device__ __forceinline__ long act_op(const int4& a0, const int4& a1, int j) {
  return (j == 0) ? lo64(a0) : (j == 1) ? hi64(a0) : (j == 2) ? lo64(a1) : hi64(a1);
}

// B operand of a weight tile for block j of the quad.  Q8_0: the 8 codes.  Q4_0: the 8
// nibbles as unsigned bytes 0..15 (low nibbles = elements 4g..4g+3, high = 4g+16..4g+19);
// the -8 offset of every code is added by a second MFMA against a constant -8 operand.
// Bits 0..3 of x to bit 0 of bytes 0..3 (the four shifted copies never overlap or carry).
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return (x * 0x00204081u) & 0x01010101u; }
// Bit pairs 0..3 of x to bits 0-1 of bytes 0..3.
__device__ __forceinline__ uint32_t spread2(uint32_t x) {
  return (x & 3u) | ((x & 0xCu) << 6) | ((x & 0x30u) << 12) | ((x & 0xC0u) << 18);
}
// Four 6-bit codes c (one per byte, 0..63) to the int8 bytes c - 32: flipping bit 5 gives the
// 6-bit two's complement of c - 32, whose sign bit 5 is then copied into bits 6 and 7.
__device__ __forceinline__ uint32_t minus32_6bit(uint32_t v) {
  const uint32_t t = v ^ 0x20202020u, s = t & 0x20202020u;
  return t | (s << 1) | (s << 2);
}

// K-quant tiles: the code bytes of block j for this lane, Q4_K/Q5_K unsigned (0..15, 0..31),
// Q6_K signed (-32..31), low 4 bytes elements 4g..4g+3 and high 4 bytes elements 4g+16..4g+19.
template <int FMT>
__device__ __forceinline__ long w_op(const int4& w0, const int4& w1, int j) {
  if (FMT == KD_FMT_Q8_0) return (j == 0) ? lo64(w0) : (j == 1) ? hi64(w0) : (j == 2) ? lo64(w1) : hi64(w1);
  const uint32_t word = (j == 0) ? (uint32_t)w0.x : (j == 1) ? (uint32_t)w0.y : (j == 2) ? (uint32_t)w0.z : (uint32_t)w0.w;
  uint32_t lo = word & 0x0F0F0F0Fu;
  uint32_t hi = (word >> 4) & 0x0F0F0F0Fu;
  if (FMT == KD_FMT_Q5_K) {  // byte j of w1.x: bit i = fifth bit of element 4g+i, bit 4+i of 4g+16+i
    const uint32_t hb = ((uint32_t)w1.x >> (8 * j)) & 0xFFu;
    lo |= spread4(hb & 15u) << 4;
    hi |= spread4(hb >> 4) << 4;
  } else if (FMT == KD_FMT_Q6_K) {  // 16 bits per block: pairs of elements 4g+i, then 4g+16+i
    const uint32_t hw = ((j < 2 ? (uint32_t)w1.x : (uint32_t)w1.y) >> (16 * (j & 1))) & 0xFFFFu;
    lo = minus32_6bit(lo | (spread2(hw & 0xFFu) << 4));
    hi = minus32_6bit(hi | (spread2(hw >> 8) << 4));
  }
  return (long)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// Exact int32 block dots for block j: S = sum_k x_k * q_k.  For Q4_0, q_k = nibble_k - 8, so
// S = sum_k x_k * nibble_k + sum_k x_k * (-8): the second term is one more MFMA against the
// constant operand -8 (all bytes 0xF8), accumulated into the first (integers: exact).
template <int FMT>
__device__ __forceinline__ v4i block_dots(long A, long Bw) {
  const v4i zero = {0, 0, 0, 0};
  v4i S = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, Bw, zero, 0, 0, 0);
  if (FMT == KD_FMT_Q4_0) S = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, (long)0xF8F8F8F8F8F8F8F8ull, S, 0, 0, 0);
  return S;
}

// Q4_0 offset term of one block, sum_k x_k * (-8) for every activation row: it depends on the
// activations only, so a quad's four offsets serve all the workgroup's row groups.
__device__ __forceinline__ v4i block_offset(long A) {
  const v4i zero = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(A, (long)0xF8F8F8F8F8F8F8F8ull, zero, 0, 0, 0);
}

__device__ __forceinline__ float half_bits(uint32_t hw, int hi) {
  return __half2float(__ushort_as_half((unsigned short)(hi ? (hw >> 16) : (hw & 0xFFFF))));
}

constexpr int kWeightAux = kWeightNT ? 2 : 0;

// One weight tile of a wave's stream: 16 bytes per lane (two for Q8_0; Q5_K and Q6_K add
// 4 and 8 bytes of upper code bits in w1).
template <int FMT>
struct WStage {
  int4 w0, w1;
};

// Issue the loads of one tile (an invalid tile reads zeros with no traffic).
template <int FMT>
__device__ __forceinline__ void wstage_load(WStage<FMT>& st, __amdgpu_buffer_rsrc_t rw, uint32_t tile, bool valid,
                                            int lane) {
  constexpr uint32_t TILE = tile_qs_bytes(FMT);
  const uint32_t wo = valid ? tile * TILE + lane * 16 : kOOB;
  st.w0 = buf16<kWeightAux>(rw, wo);
  if (FMT == KD_FMT_Q8_0) {
    st.w1 = buf16<kWeightAux>(rw, valid ? wo + 1024 : kOOB);
  } else if (FMT == KD_FMT_Q5_K) {
    st.w1 = make_int4((int)buf4u<kWeightAux>(rw, valid ? tile * TILE + 1024 + lane * 4 : kOOB), 0, 0, 0);
  } else if (FMT == KD_FMT_Q6_K) {
    const uint2 h = buf8<kWeightAux>(rw, valid ? tile * TILE + 1024 + lane * 8 : kOOB);
    st.w1 = make_int4((int)h.x, (int)h.y, 0, 0);
  } else {
    st.w1 = st.w0;
  }
}

// LDS slice of one wave (bytes): activation scales [16][QW] float4 and weight scales
// [RG][QW][16 columns] float4, converted to fp32 once when staged.
__host__ __device__ constexpr int mmvq_wave_lds(int QW, int RG) { return 16 * QW * 16 + RG * QW * 256; }

// grid (ceil(NR / RG), n_groups); block = nw waves.  A workgroup owns RG consecutive row
// groups.  Wave w owns quads [q0, q1) = [w*QW, min(NQ, w*QW + QW)) of every one of them (a
// partition that depends on NQ only).  It first fetches, with few wide loads, the scales
// its tiles share -- the weight scales of its RG x QW tiles (8 bytes per lane covering four
// tiles) and the activation scales of its quads -- into its own LDS slice, and then streams
// the weight tiles quad by quad through a depth-D register ring, so tile t is computed while
// tiles t+1 .. t+D-1 are in flight; the activation operands of a quad are loaded once for
// its RG tiles, one quad ahead.  Loads are branch-free (out-of-range tiles read zeros and
// add exactly zero).  The waves' partial sums are added in wave order through LDS.  Per output, the fp32
// sequence is: the blocks of the wave's quads in ascending order, then the waves in
// ascending order -- a function of k alone.
// Dynamic LDS: nw wave slices, then [nw][RG][4][64] floats, then (fused epilogues) the
// workgroup's outputs [RG * 16][16].
template <int FMT, int QW, int NS, int RG, int EPI, bool DEBUG, bool XG = false>
__device__ __forceinline__ void mmvq_body(const MmvqArgs& a) {
  constexpr int NT = RG * QW;
  constexpr int D0 = EPI == EPI_RESNORM ? kDepthRN : RG > 1 ? kDepthRG : FMT == KD_FMT_Q8_0 ? kDepthQ8 : kDepthQ4;
  constexpr int D = D0 < NT ? D0 : NT;
  const int e = blockIdx.y;
  const bool xg = XG && e >= a.n_groups;  // a slice of the extra matrix, on all B rows
  int nrows = a.B;
  // row split (add + RMSNorm products): this workgroup's rows start at activation row b0
  int b0 = 0;
  if (EPI == EPI_RESNORM && a.row_split) {
    b0 = (int)blockIdx.z * a.row_split;
    nrows = min(a.row_split, a.B - b0);
  }
  const int32_t* act_row = nullptr;
  const int32_t* out_row = nullptr;
  // grouped: the row map's entries for this lane's operand rows are read together with the
  // group's count (the map holds 16 entries per group, so the reads stay in bounds; entries
  // past the count are masked below)
  const int lane0 = threadIdx.x & 63;
  int32_t ar_a = 0, ar_s = 0;
  if (a.count && !xg) {
    ar_a = a.act_row[e * 16 + mfma_row_b(lane0 & 15)];
    ar_s = a.act_row[e * 16 + mfma_row_b(lane0 >> 2)];
    nrows = a.count[e];
    if (nrows <= 0) return;
    act_row = a.act_row + e * 16;
    out_row = a.out_row + e * 16;
  }
  extern __shared__ float smem[];
  const int nw = blockDim.x >> 6;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, n = lane & 15;
  const int NQ = a.NQ;
  const int q0 = w * QW;
  const int q1 = min(NQ, q0 + QW);
  const int rg0 = blockIdx.x * RG;

  const __amdgpu_buffer_rsrc_t rw = xg ? make_rsrc(a.x_wq, a.x_w_bytes) : make_rsrc(a.wq, a.w_bytes);
  const __amdgpu_buffer_rsrc_t rd = xg ? make_rsrc(a.x_wd, a.x_d_bytes) : make_rsrc(a.wd, a.d_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xq, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.xd, a.xd_bytes);
  const uint32_t gtile = (uint32_t)((size_t)(xg ? e - a.n_groups : e) * (size_t)a.w_group_tiles);
  // A operand of lane n: operand row n = activation row mfma_row_b(n) (rows past the live
  // rows read zeros)
  const int bn = mfma_row_b(n);
  const uint32_t a_off = (bn < nrows) ? (uint32_t)(act_row ? ar_a : b0 + bn) * (uint32_t)NQ * 128u + g * 32 : kOOB;

  char* slice = reinterpret_cast<char*>(smem) + (size_t)w * mmvq_wave_lds(QW, RG);
  float* dxw = reinterpret_cast<float*>(slice);  // [16][QW] float4
  char* dww = slice + 16 * QW * 16;              // [RG][QW][16 columns] float4 (fp32 scales)

  // ---- fetches shared by the wave's tiles, in the order they are consumed (loads complete in
  // issue order): activation scales, weight scales
  // activation scales: operand rows 0..15 x quads [q0, q0 + QW), float4 per (row, quad);
  // lane l fetches (operand row l/4, quads (l%4) + 4i)
  constexpr int NDX = (QW + 3) / 4;
  int4 dxv[NDX];
  if (!DEBUG) {
    const int r = lane >> 2, p = lane & 3, br = mfma_row_b(r);
    const uint32_t row_base = (br < nrows) ? (uint32_t)(act_row ? ar_s : b0 + br) * (uint32_t)NQ * 16u : kOOB;
#pragma unroll
    for (int i = 0; i < NDX; ++i) {
      const int q = q0 + 4 * i + p;
      const uint32_t off = (4 * i + p < QW && q < q1 && row_base != kOOB) ? row_base + (uint32_t)q * 16u : kOOB;
      dxv[i] = buf16<0>(rs, off);
    }
  }
  // weight scales: for row group r, the wave's QW tiles are consecutive (128 B each); lane l
  // fetches 8 bytes at 8l + 512i (K-quants: the 8 bytes of column l % 16 of tile 4i + l / 16,
  // and that column's 4 bytes of super-block scales)
  constexpr int NDW = (QW + 3) / 4;
  constexpr bool KQ = fmt_is_kq(FMT);
  constexpr uint32_t TD = tile_d_bytes(FMT);
  uint2 dwv[RG][NDW];
  uint32_t dsv[RG][NDW];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int i = 0; i < NDW; ++i) {
      const int j = 4 * i + (lane >> 4);  // the tile these 8 bytes belong to
      const bool valid = j < QW && q0 + j < q1 && rg0 + r < a.NR;
      const uint32_t tile = gtile + (uint32_t)(rg0 + r) * NQ + q0 + j;
      dwv[r][i] = buf8<kWeightAux>(rd, valid ? tile * TD + (lane & 15) * 8 : kOOB);
      dsv[r][i] = KQ ? buf4u<kWeightAux>(rd, valid ? tile * TD + 128 + (lane & 15) * 4 : kOOB) : 0u;
    }

  // ---- D weight tiles in flight (quad j = t / RG, row group r = t % RG)
  WStage<FMT> st[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int j = i / RG, r = i % RG;
    wstage_load<FMT>(st[i], rw, gtile + (uint32_t)(rg0 + r) * NQ + q0 + j, q0 + j < q1 && rg0 + r < a.NR, lane);
  }
  // the first two quads' activation operands (one quad ahead afterwards)
  int4 ax0[2], ax1[2];
#pragma unroll
  for (int j = 0; j < 2 && j < QW; ++j) {
    const uint32_t ao = (q0 + j < q1 && a_off != kOOB) ? a_off + (uint32_t)(q0 + j) * 128u : kOOB;
    ax0[j] = buf16<0>(rx, ao);
    ax1[j] = buf16<0>(rx, ao == kOOB ? kOOB : ao + 16);
  }
  __builtin_amdgcn_sched_barrier(0);  // every prologue load is issued before anything waits

  // ---- the shared fetches into this wave's LDS slice (each waits on its own loads only)
  if (!DEBUG) {
    const int r = lane >> 2, p = lane & 3;
#pragma unroll
    for (int i = 0; i < NDX; ++i)
      if (4 * i + p < QW) *reinterpret_cast<int4*>(dxw + (r * QW + 4 * i + p) * 4) = dxv[i];
  }
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int i = 0; i < NDW; ++i) {
      const int j = 4 * i + (lane >> 4);
      if (j < QW && KQ)  // raw bytes: scale/min pairs, then d and dmin (decoded per tile)
        *reinterpret_cast<int4*>(dww + ((r * QW + j) * 16 + (lane & 15)) * 16) =
            make_int4((int)dwv[r][i].x, (int)dwv[r][i].y, (int)dsv[r][i], 0);
      else if (j < QW)
        *reinterpret_cast<float4*>(dww + ((r * QW + j) * 16 + (lane & 15)) * 16) =
            make_float4(half_bits(dwv[r][i].x, 0), half_bits(dwv[r][i].x, 1), half_bits(dwv[r][i].y, 0),
                        half_bits(dwv[r][i].y, 1));
    }

  // ---- the stream, fully unrolled (no loop back-edge, so every wait is exact): tile t =
  // (quad j = t / RG, row group r = t % RG) is computed from stage t % D, which is then
  // refilled with tile t + D.
  float acc[RG][4];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[r][s] = 0.0f;
  float4 dx[4];
  v4i qoff[4];  // Q4_0, RG > 1: the current quad's offset terms
  v4i xsum[4];  // Q4_K, Q5_K: the current quad's activation block sums (for the mins)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int j = t / RG, r = t % RG;
    WStage<FMT>& cur = st[t % D];
    const int q = q0 + j;
    const bool live = q < q1;
    if (!DEBUG && r == 0) {
#pragma unroll
      for (int s = 0; s < NS; ++s) dx[s] = *reinterpret_cast<const float4*>(dxw + ((4 * g + s) * QW + j) * 4);
    }
    const int4 A0 = ax0[j & 1], A1 = ax1[j & 1];
    if (FMT == KD_FMT_Q4_0 && RG > 1 && r == 0) {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) qoff[jb] = block_offset(act_op(A0, A1, jb));
    }
    if constexpr (KQ) {
      // K-quant tile.  Q4_K/Q5_K: y += dx (d sc_j S_j - dmin m_j X_j) with S_j the dot of the
      // unsigned codes and X_j the sum of the activation codes of block j (one more MFMA
      // against an all-ones operand, once per quad).  Q6_K: y += dx d (sc_2j S'_j + sc_2j+1 S''_j)
      // with S' and S'' the dots over the block's two 16-value halves (the weight operand with
      // its other half zeroed).  Every integer is exact; the fp32 terms run in block order.
      if (FMT != KD_FMT_Q6_K && r == 0) {
        const v4i zero = {0, 0, 0, 0};
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
          xsum[jb] = __builtin_amdgcn_mfma_i32_16x16x32_i8(act_op(A0, A1, jb), (long)0x0101010101010101ull, zero, 0, 0,
                                                           0);
      }
      const int4 raw = *reinterpret_cast<const int4*>(dww + ((r * QW + j) * 16 + n) * 16);
      const float dsup = half_bits((uint32_t)raw.z, 0), dmin = half_bits((uint32_t)raw.z, 1);
      v4i Sa[4], Sc[4];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const v4i zero = {0, 0, 0, 0};
        const long A = act_op(A0, A1, jb), Bw = w_op<FMT>(cur.w0, cur.w1, jb);
        if (FMT == KD_FMT_Q6_K) {
          Sa[jb] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, (long)((uint64_t)Bw & 0xFFFFFFFFull), zero, 0, 0, 0);
          Sc[jb] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, (long)((uint64_t)Bw & 0xFFFFFFFF00000000ull), zero, 0, 0, 0);
        } else {
          Sa[jb] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, Bw, zero, 0, 0, 0);
        }
      }
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const uint32_t word = (uint32_t)(jb < 2 ? raw.x : raw.y) >> (16 * (jb & 1));
        if (FMT == KD_FMT_Q6_K) {
          const float e0 = dsup * (float)(int)(int8_t)(word & 0xFFu);
          const float e1 = dsup * (float)(int)(int8_t)((word >> 8) & 0xFFu);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const float dxs = f4_get(dx[s], jb);
            acc[r][s] = fmaf(e0 * dxs, (float)Sa[jb][s], acc[r][s]);
            acc[r][s] = fmaf(e1 * dxs, (float)Sc[jb][s], acc[r][s]);
          }
        } else {
          const float es = dsup * (float)(word & 0xFFu), em = dmin * (float)((word >> 8) & 0xFFu);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const float dxs = f4_get(dx[s], jb);
            acc[r][s] = fmaf(es * dxs, (float)Sa[jb][s], acc[r][s]);
            acc[r][s] = fmaf(-(em * dxs), (float)xsum[jb][s], acc[r][s]);
          }
        }
      }
    } else {
    // tiles past the wave's quads have zero weight and activation scales: they add exact zeros
    const float4 dw = *reinterpret_cast<const float4*>(dww + ((r * QW + j) * 16 + n) * 16);
    // the tile's four block products first (independent: their latencies overlap), then the
    // fp32 epilogue in block order
    v4i Sb[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      // Q4_0 with several row groups: nibble dots accumulated onto the quad's cached offsets
      // (the same exact integers as block_dots)
      Sb[jb] = (FMT == KD_FMT_Q4_0 && RG > 1)
                   ? __builtin_amdgcn_mfma_i32_16x16x32_i8(act_op(A0, A1, jb), w_op<FMT>(cur.w0, cur.w1, jb),
                                                           qoff[jb], 0, 0, 0)
                   : block_dots<FMT>(act_op(A0, A1, jb), w_op<FMT>(cur.w0, cur.w1, jb));
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const v4i S = Sb[jb];
      if (DEBUG) {
        const int blk = 4 * q + jb;
        const int row = (rg0 + r) * 16 + n;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int b = g + 4 * s;
          if (live && b < nrows && row < a.n_out && blk < a.kblocks)
            a.debug_S[((size_t)b * a.n_out + row) * a.kblocks + blk] = S[s];
        }
      } else {
        const float dwj = f4_get(dw, jb);
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[r][s] = fmaf(dwj * f4_get(dx[s], jb), (float)S[s], acc[r][s]);
      }
    }
    }
    if (r == RG - 1 && j + 2 < QW) {  // this quad's operand slot now takes quad j + 2
      const uint32_t ao = (q0 + j + 2 < q1 && a_off != kOOB) ? a_off + (uint32_t)(q0 + j + 2) * 128u : kOOB;
      ax0[j & 1] = buf16<0>(rx, ao);
      ax1[j & 1] = buf16<0>(rx, ao == kOOB ? kOOB : ao + 16);
    }
    if (t + D < NT) {
      const int j2 = (t + D) / RG, r2 = (t + D) % RG;
      wstage_load<FMT>(cur, rw, gtile + (uint32_t)(rg0 + r2) * NQ + q0 + j2, q0 + j2 < q1 && rg0 + r2 < a.NR, lane);
    }
    if (RG > 1) __builtin_amdgcn_sched_barrier(0);  // tiles do not interleave (registers)
  }
  if (DEBUG) return;

  constexpr bool kNormEpi = EPI == EPI_SWIGLU || EPI == EPI_ROPE;  // may take a normalised input
  float ssv[kNormPerLane];
  const bool norm = kNormEpi && a.norm_ss != nullptr;

  float* red = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + (size_t)nw * mmvq_wave_lds(QW, RG));
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int s = 0; s < 4; ++s) red[((w * RG + r) * 4 + s) * 64 + lane] = acc[r][s];
  __syncthreads();
  if (EPI == EPI_PLAIN) {
    for (int t = threadIdx.x; t < RG * NS * 64; t += blockDim.x) {
      const int r = t / (NS * 64), s = (t >> 6) % NS, l = t & 63;
      const float v = sum_waves<RG>(red, nw, r, s, l);
      const int b = (l >> 4) + 4 * s;
      const int row = (rg0 + r) * 16 + (l & 15);
      if (b < nrows && row < a.n_out) {
        const int orow = out_row ? out_row[b] : b;
        float o = v;
        if (a.mo_y) {
          float acc = 0.0f;
          for (int k = 0; k < a.mo_K; ++k)
            acc = fmaf(a.mo_p[b * a.mo_K + k], a.mo_y[(size_t)(b * a.mo_K + k) * a.n_out + row], acc);
          o = acc + v;
        }
        a.y[(size_t)orow * a.ldy + row] = o;
      }
    }
    return;
  }
  // normalised input: this thread's first row's block sums, in flight while the outputs are
  // assembled (unconditional -- with no sums every load reads zero -- since a branch lets the
  // compiler sink earlier work below it and hold its registers across the loads)
  if (kNormEpi) norm_ss_load(a, threadIdx.x, nrows, ssv);
  // fused epilogues: the workgroup's outputs outv[row in workgroup][activation row]
  float* outv = red + nw * RG * 256;
  for (int t = threadIdx.x; t < RG * NS * 64; t += blockDim.x) {
    const int r = t / (NS * 64), s = (t >> 6) % NS, l = t & 63;
    const float v = sum_waves<RG>(red, nw, r, s, l);
    outv[(r * 16 + (l & 15)) * 16 + (l >> 4) + 4 * s] = v;
  }
  __syncthreads();
  // 8 lanes per (activation row, 32-element block); the loop steps by whole waves, so the 8
  // lanes of a group stay together (small-k launches have a single wave)
  for (int t = threadIdx.x; t < 8 * nrows; t += blockDim.x) {
    const int bq = t >> 3, sub = t & 7;
    float inv = 1.0f;  // normalised input: 1/rms of activation row bq
    if (norm) {
      if (t == (int)threadIdx.x) {
        inv = norm_inv(a, ssv);
      } else {  // a second row of a single-wave workgroup
        float v2[kNormPerLane];
        norm_ss_load(a, t, nrows, v2);
        inv = norm_inv(a, v2);
      }
    }
    if (EPI == EPI_SWIGLU) {
      // rows 0..31 of the workgroup: gate rows 32m..32m+31; rows 32..63: the same up rows
      const int m = blockIdx.x, F = a.n_out / 2;
      // the output rows, their width and this workgroup's output block (extra-matrix slice c:
      // block c F / 32 + m of rows F x_groups wide)
      int8_t* const oq = xg ? a.x_qs : a.epi_qs;
      float* const od = xg ? a.x_qd : a.epi_qd;
      const int Fo = xg ? F * a.x_groups : F, mo = xg ? (e - a.n_groups) * (F / 32) + m : m;
      const int NQo = n_quads(Fo), nbpo = NQo * 4;
      float av[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int i = 4 * sub + e2;
        float gv = outv[i * 16 + bq], uv = outv[(32 + i) * 16 + bq];
        if (norm) {
          gv *= inv;
          uv *= inv;
        }
        av[e2] = (gv / (1.0f + expf(-gv))) * uv;
      }
      const int orow = out_row ? out_row[bq] : bq;  // grouped (experts): the row's (row, rank) pair
      quant4_lane8(make_float4(av[0], av[1], av[2], av[3]), sub, true,
                   oq + ((size_t)orow * NQo + (mo >> 2)) * 128 + (mo & 3) * 8, od + (size_t)orow * nbpo + mo);
      if (mo == Fo / 32 - 1)  // zero blocks past Fo (only when Fo is not a multiple of 128)
        for (int blk = Fo / 32; blk < nbpo; ++blk)
          quant4_lane8(make_float4(0.0f, 0.0f, 0.0f, 0.0f), sub, true,
                       oq + ((size_t)orow * NQo + (blk >> 2)) * 128 + (blk & 3) * 8, od + (size_t)orow * nbpo + blk);
    } else if (EPI == EPI_RESNORM) {
      // the workgroup's 32 rows are block m of the residual row: x1 = res + y (activation
      // row bg = b0 + bq)
      const int m = blockIdx.x, Dn = a.n_out, nblk = Dn / 32, bg = b0 + bq;
      const int NQo = n_quads(Dn), nbpo = NQo * 4;
      const size_t o = (size_t)bg * a.epi_ld + 32 * m + 4 * sub;
      const float4 xr = *reinterpret_cast<const float4*>(a.epi_res + o);
      const float4 gn = *reinterpret_cast<const float4*>(a.epi_gain + 32 * m + 4 * sub);
      const float* ov = outv + (4 * sub) * 16 + bq;
      const float4 v = make_float4(xr.x + ov[0], xr.y + ov[16], xr.z + ov[32], xr.w + ov[48]);
      *reinterpret_cast<float4*>(a.epi_x1 + o) = v;
      float ss = v.x * v.x;
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
      ss = group8_sum(ss);
      if (sub == 0) a.epi_ss[(size_t)bg * nblk + m] = ss;
      quant4_lane8(make_float4(v.x * gn.x, v.y * gn.y, v.z * gn.z, v.w * gn.w), sub, true,
                   a.epi_qs + ((size_t)bg * NQo + (m >> 2)) * 128 + (m & 3) * 8, a.epi_qd + (size_t)bg * nbpo + m);
      if (m == nblk - 1)  // zero blocks past the row (only when it is not a multiple of 128)
        for (int blk = nblk; blk < nbpo; ++blk)
          quant4_lane8(make_float4(0.0f, 0.0f, 0.0f, 0.0f), sub, true,
                       a.epi_qs + ((size_t)bg * NQo + (blk >> 2)) * 128 + (blk & 3) * 8,
                       a.epi_qd + (size_t)bg * nbpo + blk);
    } else {
      // 16 rows = 8 RoPE pairs (i, i + hd/2) of one head, packed adjacently
      const int hd = a.epi_hd, half = hd / 2, H = a.epi_H, G = a.epi_G;
      const int row0 = rg0 * 16, hh = row0 / hd, i = (row0 % hd) / 2 + sub;
      float x0 = outv[(2 * sub) * 16 + bq], x1 = outv[(2 * sub + 1) * 16 + bq];
      if (norm) {
        x0 *= inv;
        x1 *= inv;
      }
      const int pos = a.epi_rc.pos[bq];
      if (hh < H + G) {
        const float2 cs = a.epi_cs ? make_float2(a.epi_cs[2 * (bq * half + i)], a.epi_cs[2 * (bq * half + i) + 1])
                                   : rope_cs(pos, i, hd, a.epi_base);
        const float y0 = fmaf(x0, cs.x, -(x1 * cs.y));
        const float y1 = fmaf(x0, cs.y, x1 * cs.x);
        if (hh < H) {
          float* qr = a.epi_q + (size_t)bq * a.epi_ldq + (size_t)hh * hd;
          qr[i] = y0;
          qr[i + half] = y1;
        } else {
          const size_t o = ((size_t)(hh - H) * a.epi_capacity + pos) * hd;
          if (a.epi_kv8) {
            uint8_t* K = static_cast<uint8_t*>(a.epi_rc.k[bq]) + o;
            K[i] = (uint8_t)f32_to_e4m3(y0);
            K[i + half] = (uint8_t)f32_to_e4m3(y1);
          } else {
            __half* K = static_cast<__half*>(a.epi_rc.k[bq]) + o;
            K[i] = __float2half_rn(y0);
            K[i + half] = __float2half_rn(y1);
          }
        }
      } else if (hh < H + 2 * G) {
        const size_t o = ((size_t)(hh - H - G) * a.epi_capacity + pos) * hd;
        if (a.epi_kv8) {
          uint8_t* V = static_cast<uint8_t*>(a.epi_rc.v[bq]) + o;
          V[i] = (uint8_t)f32_to_e4m3(x0);
          V[i + half] = (uint8_t)f32_to_e4m3(x1);
        } else {
          __half* V = static_cast<__half*>(a.epi_rc.v[bq]) + o;
          V[i] = __float2half_rn(x0);
          V[i + half] = __float2half_rn(x1);
        }
      } else {  // output-gate rows (gated layers): stored as they are, after v in the row
        float* gr = a.epi_q + (size_t)bq * a.epi_ldq + (size_t)hh * hd;
        gr[i] = x0;
        gr[i + half] = x1;
      }
    }
  }
}

// The product kernel.  GRP (grouped launches, 4 accumulator slots): each workgroup runs the
// copy of the body with as many slots as its group's rows need (slot s holds rows 4s .. 4s+3),
// so a group of few rows does only its own rows' epilogue work; every live output takes the
// same operations in every copy.
template <int FMT, int QW, int NS, int RG, int EPI, bool DEBUG, bool GRP = false>
__global__ __launch_bounds__(1024) void mmvq_kernel(MmvqArgs a) {
  if constexpr (GRP) {
    const int rows = (int)blockIdx.y >= a.n_groups ? a.B : a.count[blockIdx.y];
    if (rows <= 4)
      mmvq_body<FMT, QW, 1, RG, EPI, DEBUG, true>(a);
    else if (rows <= 8)
      mmvq_body<FMT, QW, 2, RG, EPI, DEBUG, true>(a);
    else if (rows <= 12)
      mmvq_body<FMT, QW, 3, RG, EPI, DEBUG, true>(a);
    else
      mmvq_body<FMT, QW, 4, RG, EPI, DEBUG, true>(a);
  } else {
    mmvq_body<FMT, QW, NS, RG, EPI, DEBUG>(a);
  }
}

// Quads per wave: about NQ / 4 (four waves per workgroup), between 2 and kWaveQuads,
// and enough that at most 16 waves cover NQ; then balanced (the smallest QW giving the same
// wave count).  Waves per workgroup: ceil(NQ / QW).  Both depend on the matrix's k only.
static int mmvq_qw(int NQ, int want_quads = kWaveQuads) {
  int qw = ceil_div(NQ, 16);  // at most 16 waves; QW <= 8 covers k <= 16384
  want_quads = NQ / 4 < want_quads ? (NQ / 4 > 2 ? NQ / 4 : 2) : want_quads;
  const int want = NQ < want_quads ? NQ : want_quads;
  qw = qw > want ? qw : want;
  const int nw = ceil_div(NQ, qw);
  return ceil_div(NQ, nw);
}

template <int FMT, int QW, int NS, int RG, int EPI>
static void launch_mmvq_qn(const MmvqArgs& a, int n_groups, hipStream_t st) {
  const int nw = ceil_div(a.NQ, QW);
  dim3 grid(ceil_div(a.NR, RG), n_groups, a.row_split ? ceil_div(a.B, a.row_split) : 1);
  const size_t slices = (size_t)nw * mmvq_wave_lds(QW, RG);
  const size_t red_shm = (size_t)nw * RG * 256 * sizeof(float);
  const size_t out_shm = EPI == EPI_PLAIN ? 0 : (size_t)RG * 256 * sizeof(float);
  if constexpr (EPI == EPI_PLAIN && !fmt_is_kq(FMT)) {
    if (a.debug_S) {
      mmvq_kernel<FMT, QW, 4, RG, EPI_PLAIN, true><<<grid, 64 * nw, slices, st>>>(a);
      return;
    }
  }
  // (the grouped down product, k = expert_ffn, keeps the one body: its epilogue is small)
  if constexpr (NS == 4 && EPI == EPI_SWIGLU && (FMT == KD_FMT_Q4_0 || FMT == KD_FMT_Q8_0)) {
    if (a.count) {
      mmvq_kernel<FMT, QW, NS, RG, EPI, false, true><<<grid, 64 * nw, slices + red_shm + out_shm, st>>>(a);
      return;
    }
  }
  mmvq_kernel<FMT, QW, NS, RG, EPI, false><<<grid, 64 * nw, slices + red_shm + out_shm, st>>>(a);
}

template <int FMT, int QW, int RG, int EPI>
static void launch_mmvq_q(const MmvqArgs& a, int n_groups, hipStream_t st) {
  // epilogue slots: ceil(rows / 4) for the rows a workgroup takes (B, or a row split's slice;
  // rows past them are never written, so dropping their slots leaves every live output's
  // operation sequence unchanged)
  // (K-quant formats: 2 slots up to B = 8, else 4 -- two instantiations)
  const int rows = a.row_split ? a.row_split : a.B;  // rows per workgroup
  if constexpr (fmt_is_kq(FMT)) {
    if (!a.count && rows <= 8)
      launch_mmvq_qn<FMT, QW, 2, RG, EPI>(a, n_groups, st);
    else
      launch_mmvq_qn<FMT, QW, 4, RG, EPI>(a, n_groups, st);
  } else {
    const int ns = a.count ? 4 : (rows + 3) / 4;
    switch (ns) {
      case 1: return launch_mmvq_qn<FMT, QW, 1, RG, EPI>(a, n_groups, st);
      case 2: return launch_mmvq_qn<FMT, QW, 2, RG, EPI>(a, n_groups, st);
      case 3: return launch_mmvq_qn<FMT, QW, 3, RG, EPI>(a, n_groups, st);
      default: return launch_mmvq_qn<FMT, QW, 4, RG, EPI>(a, n_groups, st);
    }
  }
}

template <int FMT, int RG, int EPI>
static void launch_mmvq_t(const MmvqArgs& a, int n_groups, hipStream_t st) {
  switch (a.QW) {
    case 1: return launch_mmvq_q<FMT, 1, RG, EPI>(a, n_groups, st);
    case 2: return launch_mmvq_q<FMT, 2, RG, EPI>(a, n_groups, st);
    case 3: return launch_mmvq_q<FMT, 3, RG, EPI>(a, n_groups, st);
    case 4: return launch_mmvq_q<FMT, 4, RG, EPI>(a, n_groups, st);
    case 5: return launch_mmvq_q<FMT, 5, RG, EPI>(a, n_groups, st);
    case 6: return launch_mmvq_q<FMT, 6, RG, EPI>(a, n_groups, st);
    case 7: return launch_mmvq_q<FMT, 7, RG, EPI>(a, n_groups, st);
    default: return launch_mmvq_q<FMT, 8, RG, EPI>(a, n_groups, st);
  }
}

// The K-quant formats' launches (instantiated in mmvq_kq.hip for the products' (RG, EPI)
// pairs: (kPlainRG, EPI_PLAIN), (4, EPI_SWIGLU), (2, EPI_RESNORM), (1, EPI_ROPE)).
template <int RG, int EPI>
void launch_mmvq_kq(int fmt, const MmvqArgs& a, int n_groups, hipStream_t st);
// Repack K-quant records (rows of k / 256 records of 144 / 176 / 210 bytes) into tiles.
void launch_pack_kquant(int fmt, const uint8_t* src, int n_out, int k, uint8_t* dst_qs, uint8_t* dst_d,
                        hipStream_t st);

}  // namespace kd
