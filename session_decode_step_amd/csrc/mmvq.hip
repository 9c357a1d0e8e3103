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

// Launch shape constants (measured on MI355X; see the mmvq design notes).
constexpr bool kWeightNT = true;  // weight tiles are streamed once: non-temporal loads
constexpr int kDepthQ4 = 2;       // weight-ring depth, one row group per workgroup, Q4_0
constexpr int kDepthQ8 = 2;       // the same for Q8_0
constexpr int kDepthRG = 4;       // ring depth when a workgroup streams several row groups
constexpr int kDepthRN = 4;       // ring depth of the add + RMSNorm products (two row groups)
constexpr int kWaveQuads = 8;     // quads per wave of the plain, SwiGLU and RoPE products
constexpr int kQuadsRN = 2;       // quads per wave of the add + RMSNorm products
constexpr int kPlainRG = 1;       // row groups per workgroup of the plain product
// the largest k a product takes: 16 waves of kWaveQuads quads of 128 elements
constexpr int kMaxK = 16 * kWaveQuads * 128;

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
// DPP sum over the 8-lane group (group8_sum: every lane ends with the same value).
constexpr int kNormPerLane = 16;  // block sums per lane: rows of up to 8 * 16 * 32 = 4096

__device__ __forceinline__ void norm_ss_load(const MmvqArgs& a, int t, int nrows, float (&v)[kNormPerLane]) {
  const int bq = t >> 3, sub = t & 7;
  const int nblk = a.norm_n / 32, c = (nblk + 7) / 8;
  // no sums (plain SwiGLU): an empty range, every load reads zero without touching memory
  const __amdgpu_buffer_rsrc_t r =
      a.norm_ss ? make_rsrc(a.norm_ss, (uint32_t)(nrows * nblk * 4)) : make_rsrc(a.xd, 0u);
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
template <int FMT>
__device__ __forceinline__ long w_op(const int4& w0, const int4& w1, int j) {
  if (FMT == KD_FMT_Q8_0) return (j == 0) ? lo64(w0) : (j == 1) ? hi64(w0) : (j == 2) ? lo64(w1) : hi64(w1);
  const uint32_t word = (j == 0) ? (uint32_t)w0.x : (j == 1) ? (uint32_t)w0.y : (j == 2) ? (uint32_t)w0.z : (uint32_t)w0.w;
  const uint32_t lo = word & 0x0F0F0F0Fu;
  const uint32_t hi = (word >> 4) & 0x0F0F0F0Fu;
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

// One weight tile of a wave's stream: 16 bytes per lane (two for Q8_0).
template <int FMT>
struct WStage {
  int4 w0, w1;
};

// Issue the loads of one tile (an invalid tile reads zeros with no traffic).
template <int FMT>
__device__ __forceinline__ void wstage_load(WStage<FMT>& st, __amdgpu_buffer_rsrc_t rw, uint32_t tile, bool valid,
                                            int lane) {
  constexpr int TILE = FMT == KD_FMT_Q8_0 ? kTileQ8 : kTileQ4;
  const uint32_t wo = valid ? tile * TILE + lane * 16 : kOOB;
  st.w0 = buf16<kWeightAux>(rw, wo);
  st.w1 = (FMT == KD_FMT_Q8_0) ? buf16<kWeightAux>(rw, valid ? wo + 1024 : kOOB) : st.w0;
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
template <int FMT, int QW, int NS, int RG, int EPI, bool DEBUG>
__global__ __launch_bounds__(1024) void mmvq_kernel(MmvqArgs a) {
  constexpr int NT = RG * QW;
  constexpr int D0 = EPI == EPI_RESNORM ? kDepthRN : RG > 1 ? kDepthRG : FMT == KD_FMT_Q8_0 ? kDepthQ8 : kDepthQ4;
  constexpr int D = D0 < NT ? D0 : NT;
  const int e = blockIdx.y;
  int nrows = a.B;
  const int32_t* act_row = nullptr;
  const int32_t* out_row = nullptr;
  if (a.count) {
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

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wq, a.w_bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.wd, a.d_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.xq, a.x_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.xd, a.xd_bytes);
  const uint32_t gtile = (uint32_t)((size_t)e * (size_t)a.w_group_tiles);
  // A operand of lane n: operand row n = activation row mfma_row_b(n) (rows past the live
  // rows read zeros)
  const int bn = mfma_row_b(n);
  const uint32_t a_off = (bn < nrows) ? (uint32_t)(act_row ? act_row[bn] : bn) * (uint32_t)NQ * 128u + g * 32 : kOOB;

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
    const uint32_t row_base = (br < nrows) ? (uint32_t)(act_row ? act_row[br] : br) * (uint32_t)NQ * 16u : kOOB;
#pragma unroll
    for (int i = 0; i < NDX; ++i) {
      const int q = q0 + 4 * i + p;
      const uint32_t off = (4 * i + p < QW && q < q1 && row_base != kOOB) ? row_base + (uint32_t)q * 16u : kOOB;
      dxv[i] = buf16<0>(rs, off);
    }
  }
  // weight scales: for row group r, the wave's QW tiles are consecutive (128 B each); lane l
  // fetches 8 bytes at 8l + 512i
  constexpr int NDW = (QW + 3) / 4;
  uint2 dwv[RG][NDW];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int i = 0; i < NDW; ++i) {
      const int j = 4 * i + (lane >> 4);  // the tile these 8 bytes belong to
      const bool valid = j < QW && q0 + j < q1 && rg0 + r < a.NR;
      const uint32_t tile = gtile + (uint32_t)(rg0 + r) * NQ + q0 + j;
      dwv[r][i] = buf8<kWeightAux>(rd, valid ? tile * 128 + (lane & 15) * 8 : kOOB);
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
      if (j < QW)
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
    for (int t = threadIdx.x; t < RG * 256; t += blockDim.x) {
      const int r = t >> 8, s = (t >> 6) & 3, l = t & 63;
      float v = red[(r * 4 + s) * 64 + l];
      for (int ww = 1; ww < nw; ++ww) v += red[((ww * RG + r) * 4 + s) * 64 + l];  // fixed wave order
      const int b = (l >> 4) + 4 * s;
      const int row = (rg0 + r) * 16 + (l & 15);
      if (b < nrows && row < a.n_out) {
        const int orow = out_row ? out_row[b] : b;
        a.y[(size_t)orow * a.ldy + row] = v;
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
  for (int t = threadIdx.x; t < RG * 256; t += blockDim.x) {
    const int r = t >> 8, s = (t >> 6) & 3, l = t & 63;
    float v = red[(r * 4 + s) * 64 + l];
    for (int ww = 1; ww < nw; ++ww) v += red[((ww * RG + r) * 4 + s) * 64 + l];  // fixed wave order
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
      const int NQo = n_quads(F), nbpo = NQo * 4;
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
                   a.epi_qs + ((size_t)orow * NQo + (m >> 2)) * 128 + (m & 3) * 8, a.epi_qd + (size_t)orow * nbpo + m);
      if (m == F / 32 - 1)  // zero blocks past F (only when F is not a multiple of 128)
        for (int blk = F / 32; blk < nbpo; ++blk)
          quant4_lane8(make_float4(0.0f, 0.0f, 0.0f, 0.0f), sub, true,
                       a.epi_qs + ((size_t)orow * NQo + (blk >> 2)) * 128 + (blk & 3) * 8,
                       a.epi_qd + (size_t)orow * nbpo + blk);
    } else if (EPI == EPI_RESNORM) {
      // the workgroup's 32 rows are block m of the residual row: x1 = res + y
      const int m = blockIdx.x, Dn = a.n_out, nblk = Dn / 32;
      const int NQo = n_quads(Dn), nbpo = NQo * 4;
      const size_t o = (size_t)bq * a.epi_ld + 32 * m + 4 * sub;
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
      if (sub == 0) a.epi_ss[(size_t)bq * nblk + m] = ss;
      quant4_lane8(make_float4(v.x * gn.x, v.y * gn.y, v.z * gn.z, v.w * gn.w), sub, true,
                   a.epi_qs + ((size_t)bq * NQo + (m >> 2)) * 128 + (m & 3) * 8, a.epi_qd + (size_t)bq * nbpo + m);
      if (m == nblk - 1)  // zero blocks past the row (only when it is not a multiple of 128)
        for (int blk = nblk; blk < nbpo; ++blk)
          quant4_lane8(make_float4(0.0f, 0.0f, 0.0f, 0.0f), sub, true,
                       a.epi_qs + ((size_t)bq * NQo + (blk >> 2)) * 128 + (blk & 3) * 8,
                       a.epi_qd + (size_t)bq * nbpo + blk);
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
  dim3 grid(ceil_div(a.NR, RG), n_groups);
  const size_t slices = (size_t)nw * mmvq_wave_lds(QW, RG);
  const size_t red_shm = (size_t)nw * RG * 256 * sizeof(float);
  const size_t out_shm = EPI == EPI_PLAIN ? 0 : (size_t)RG * 256 * sizeof(float);
  if constexpr (EPI == EPI_PLAIN) {
    if (a.debug_S) {
      mmvq_kernel<FMT, QW, 4, RG, EPI_PLAIN, true><<<grid, 64 * nw, slices, st>>>(a);
      return;
    }
  }
  mmvq_kernel<FMT, QW, NS, RG, EPI, false><<<grid, 64 * nw, slices + red_shm + out_shm, st>>>(a);
}

template <int FMT, int QW, int RG, int EPI>
static void launch_mmvq_q(const MmvqArgs& a, int n_groups, hipStream_t st) {
  // epilogue slots: ceil(B / 4), a function of B (rows past B are never written, so
  // dropping their slots leaves every live output's operation sequence unchanged)
  const int ns = a.count ? 4 : (a.B + 3) / 4;
  switch (ns) {
    case 1: return launch_mmvq_qn<FMT, QW, 1, RG, EPI>(a, n_groups, st);
    case 2: return launch_mmvq_qn<FMT, QW, 2, RG, EPI>(a, n_groups, st);
    case 3: return launch_mmvq_qn<FMT, QW, 3, RG, EPI>(a, n_groups, st);
    default: return launch_mmvq_qn<FMT, QW, 4, RG, EPI>(a, n_groups, st);
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
  a.debug_S = debug_S;
  const size_t tiles = (size_t)(map ? map->n_groups : 1) * (map ? (size_t)map->w_group_tiles : (size_t)a.NR * a.NQ);
  a.w_bytes = (uint32_t)(tiles * (W.fmt == KD_FMT_Q8_0 ? kTileQ8 : kTileQ4));
  a.d_bytes = (uint32_t)(tiles * 128);
  const size_t rows = map ? (size_t)map->act_rows : (size_t)B;
  a.x_bytes = (uint32_t)(rows * a.NQ * 128);
  a.xd_bytes = (uint32_t)(rows * a.NQ * 16);
  return a;
}

template <int RG, int EPI>
static void launch_mmvq_fmt(const kd_weight& W, const MmvqArgs& a, int ng, hipStream_t st) {
  if (W.fmt == KD_FMT_Q8_0)
    launch_mmvq_t<KD_FMT_Q8_0, RG, EPI>(a, ng, st);
  else
    launch_mmvq_t<KD_FMT_Q4_0, RG, EPI>(a, ng, st);
}

void launch_mmvq(const kd_weight& W, const int8_t* xq, const float* xd, int B, float* y, int ldy,
                 hipStream_t st, const RowMap* map, int32_t* debug_S) {
  const MmvqArgs a = mmvq_args(W, xq, xd, B, y, ldy, map, debug_S);
  launch_mmvq_fmt<kPlainRG, EPI_PLAIN>(W, a, map ? map->n_groups : 1, st);
}

void launch_mmvq_swiglu(const kd_weight& W, const int8_t* xq, const float* xd, int B, int8_t* out_qs, float* out_d,
                        hipStream_t st, const float* norm_ss, int norm_n, float norm_eps, const RowMap* map) {
  MmvqArgs a = mmvq_args(W, xq, xd, B, nullptr, 0, map, nullptr);
  a.epi_qs = out_qs;
  a.epi_qd = out_d;
  a.norm_ss = norm_ss;
  a.norm_n = norm_n;
  a.norm_eps = norm_eps;
  a.QW = mmvq_qw(a.NQ, kWaveQuads);
  launch_mmvq_fmt<4, EPI_SWIGLU>(W, a, map ? map->n_groups : 1, st);
}

// Two row groups per workgroup (one 32-element block of the residual row); two quads per
// wave, so the workgroup count halves but the wave count does not.
void launch_mmvq_resnorm(const kd_weight& W, const int8_t* xq, const float* xd, int B, const float* res, int ld,
                         const float* gain, float* x1, int8_t* out_qs, float* out_d, float* ss, hipStream_t st) {
  MmvqArgs a = mmvq_args(W, xq, xd, B, nullptr, 0, nullptr, nullptr);
  a.QW = mmvq_qw(a.NQ, kQuadsRN);
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
  a.QW = mmvq_qw(a.NQ, kWaveQuads);
  launch_mmvq_fmt<1, EPI_ROPE>(W, a, 1, st);
}

// A product's limits: k up to kMaxK (the widest wave partition), and the tiled codes and
// scales addressable by 32-bit buffer offsets with kOOB past their end.
bool mmvq_weight_fits(int fmt, int n_out, int k) {
  if (n_out <= 0 || k <= 0 || k > kMaxK) return false;
  const size_t tiles = (size_t)n_rowgroups(n_out) * n_quads(k);
  const size_t qs = tiles * (fmt == KD_FMT_Q8_0 ? kTileQ8 : kTileQ4);
  return qs < (size_t)kOOB && tiles * 128 < (size_t)kOOB;
}
int mmvq_max_k() { return kMaxK; }

void launch_act_quant(const float* x, int B, int k, int ldx, int8_t* qs, float* d, hipStream_t st) {
  const int NQ = n_quads(k);
  act_quant_kernel<<<dim3(ceil_div(NQ * 4, 32), B), 256, 0, st>>>(x, k, ldx, NQ, qs, d);
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

extern "C" kd_status kd_mmvq_swiglu(const kd_weight* W, kd_act_q8 x, int32_t B, kd_act_q8 out, void* stream) {
  const char* who = "kd_mmvq_swiglu";
  KD_REQUIRE(W, KD_ERR_INVALID, "%s: null weight", who);
  kd_status s = check_mmvq_args(who, W, W->fmt, x, B);
  if (s != KD_OK) return s;
  KD_REQUIRE(fmt_quant(W->fmt), KD_ERR_UNSUPPORTED, "%s: format %d", who, W->fmt);
  KD_REQUIRE(W->n_out % 64 == 0, KD_ERR_UNSUPPORTED, "%s: n_out=%d is not 2F with F a multiple of 32", who,
             W->n_out);
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
  KD_REQUIRE(fmt_quant(W->fmt), KD_ERR_UNSUPPORTED, "kd_debug_block_dots: format %d", W->fmt);
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
    KD_REQUIRE(out.qs && out.d && aligned16(out.qs) && aligned16(out.d), KD_ERR_INVALID,
               "%s: output buffers null or not 16-byte aligned", who);
    launch_mmvq_swiglu(*W, x.qs, x.d, 0, out.qs, out.d, as_stream(stream), nullptr, 0, 0.0f, &map);
  } else {
    KD_REQUIRE(y && ldy >= W->n_out, KD_ERR_INVALID, "%s: null output or ldy=%d < rows per group", who, ldy);
    launch_mmvq(*W, x.qs, x.d, 0, y, ldy, as_stream(stream), &map);
  }
  return check_launch(who);
}
