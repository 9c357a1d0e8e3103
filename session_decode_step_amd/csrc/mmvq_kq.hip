// K-quant weights (Q4_K, Q5_K, Q6_K) for the mmvq products: the repack of their 256-value
// records into the MFMA tile layout, and the instantiations of the product kernel for them.
//
// What is computed: the same y = W x at m = B as for Q8_0 / Q4_0, with the weight values the
// GGUF k-quant records define (the weight types the pages require a batched decode to cover:
// hf2q ADR-040 "Quant scope"; memra-engine decode_batch.rs, exact-16 admission list with
// QT_Q4_K, QT_Q5_K and QT_Q6_K, whose products must keep each row B-invariant).
//
// How (gfx950): a record of 256 values splits into two tile quads of four 32-value blocks.
// Each block's codes stay integers in the MFMA operand -- the low nibbles as Q4_0 keeps them,
// the fifth bit (Q5_K) or the upper two bits (Q6_K, then the offset of 32 taken off in the
// byte lanes) merged in registers -- so every block dot is an exact int32.  Q4_K / Q5_K keep
// one scale and one min per block: y += d_x (d sc S - dmin m X), X the block's activation
// code sum from one more MFMA against ones.  Q6_K has a scale per 16 values: two MFMAs per
// block, one per half.  The tiles keep the records' compact scales (bytes and fp16), decoded
// per tile in registers, so the bytes streamed stay within 6 % of the records'.
#include "mmvq_impl.h"

namespace kd {

template <int FMT>
struct KqRecord;
template <>
struct KqRecord<KD_FMT_Q4_K> {
  static constexpr int bytes = 144;
};
template <>
struct KqRecord<KD_FMT_Q5_K> {
  static constexpr int bytes = 176;
};
template <>
struct KqRecord<KD_FMT_Q6_K> {
  static constexpr int bytes = 210;
};

__device__ __forceinline__ uint32_t rd16(const uint8_t* p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }

// Code of value v (0..255) of a record: Q4_K 0..15, Q5_K 0..31, Q6_K 0..63 (offset not taken off).
template <int FMT>
__device__ __forceinline__ uint32_t kq_code(const uint8_t* rec, int v) {
  if (FMT == KD_FMT_Q6_K) {
    // halves of 128 values; within a half, four runs of 32: runs 0 and 1 take the low nibbles
    // of low bytes [0, 32) and [32, 64) of the half, runs 2 and 3 their high nibbles; the
    // upper two bits of run i sit in bit pair i of upper byte l of the half
    const int hh = v >> 7, i = (v >> 5) & 3, l = v & 31;
    const uint32_t lb = rec[64 * hh + 32 * (i & 1) + l];
    const uint32_t nib = (i >> 1) ? (lb >> 4) : (lb & 15u);
    const uint32_t up = ((uint32_t)rec[128 + 32 * hh + l] >> (2 * i)) & 3u;
    return nib | (up << 4);
  }
  // Q4_K / Q5_K: runs of 64 values; code byte l of run c holds value 64c + l in its low
  // nibble and 64c + 32 + l in its high nibble
  const int c = v >> 6, h = (v >> 5) & 1, l = v & 31;
  const int off = FMT == KD_FMT_Q5_K ? 48 : 16;
  const uint32_t b = rec[off + 32 * c + l];
  uint32_t q = h ? (b >> 4) : (b & 15u);
  if (FMT == KD_FMT_Q5_K) q |= (((uint32_t)rec[16 + l] >> (2 * c + h)) & 1u) << 4;
  return q;
}

// The 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes s: sub-blocks 0..3
// in the low 6 bits of bytes j and j + 4; sub-blocks 4..7 with their low 4 bits in byte j + 4
// (scale low nibble, min high nibble) and their top 2 bits in the top bits of bytes j - 4
// (scale) and j (min).
__device__ __forceinline__ void kq_scale_min(const uint8_t* s, int j, uint32_t& sc, uint32_t& m) {
  if (j < 4) {
    sc = s[j] & 63u;
    m = s[j + 4] & 63u;
  } else {
    sc = (s[j + 4] & 15u) | ((uint32_t)(s[j - 4] >> 6) << 4);
    m = ((uint32_t)s[j + 4] >> 4) | ((uint32_t)(s[j] >> 6) << 4);
  }
}

// One thread per (row, quad): the row's four blocks of the quad into tile t = (row / 16) NQ + q.
template <int FMT>
__global__ void pack_kquant_kernel(const uint8_t* __restrict__ src, int n_out, int k, int NR, int NQ,
                                   uint8_t* __restrict__ dst_qs, uint8_t* __restrict__ dst_d) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)NR * 16 * NQ) return;
  constexpr int BS = KqRecord<FMT>::bytes;
  constexpr int TILE = tile_qs_bytes(FMT);
  const int row = (int)(idx / NQ), q = (int)(idx % NQ);
  const int n = row & 15;
  const size_t t = (size_t)(row >> 4) * NQ + q;
  const bool valid = row < n_out;
  const uint8_t* rec = src + ((size_t)row * (k / 256) + q / 2) * BS;
  uint8_t* dq = dst_qs + t * TILE;
  uint8_t* dd = dst_d + t * 192;
  const uint32_t dbits = valid ? rd16(rec + (FMT == KD_FMT_Q6_K ? 208 : 0)) : 0u;
  const uint32_t mbits = (valid && FMT != KD_FMT_Q6_K) ? rd16(rec + 2) : 0u;
  dd[128 + 4 * n + 0] = (uint8_t)(dbits & 0xFF);
  dd[128 + 4 * n + 1] = (uint8_t)(dbits >> 8);
  dd[128 + 4 * n + 2] = (uint8_t)(mbits & 0xFF);
  dd[128 + 4 * n + 3] = (uint8_t)(mbits >> 8);
  for (int j = 0; j < 4; ++j) {
    const int v0 = 128 * (q & 1) + 32 * j;  // the block's first value within the record
    uint32_t code[32];
    for (int e = 0; e < 32; ++e) code[e] = valid ? kq_code<FMT>(rec, v0 + e) : 0u;
    if (FMT == KD_FMT_Q6_K) {
      dd[8 * n + 2 * j] = valid ? rec[192 + v0 / 16] : 0;
      dd[8 * n + 2 * j + 1] = valid ? rec[192 + v0 / 16 + 1] : 0;
    } else {
      uint32_t sc = 0, m = 0;
      if (valid) kq_scale_min(rec + 4, v0 / 32, sc, m);
      dd[8 * n + 2 * j] = (uint8_t)sc;
      dd[8 * n + 2 * j + 1] = (uint8_t)m;
    }
    for (int g = 0; g < 4; ++g) {
      const int lane = 16 * g + n;
      uint32_t hb5 = 0, up_lo = 0, up_hi = 0;
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = code[4 * g + i], b = code[4 * g + 16 + i];
        dq[lane * 16 + 4 * j + i] = (uint8_t)((a & 15u) | ((b & 15u) << 4));
        hb5 |= (((a >> 4) & 1u) << i) | (((b >> 4) & 1u) << (4 + i));
        up_lo |= ((a >> 4) & 3u) << (2 * i);
        up_hi |= ((b >> 4) & 3u) << (2 * i);
      }
      if (FMT == KD_FMT_Q5_K) dq[1024 + lane * 4 + j] = (uint8_t)hb5;
      if (FMT == KD_FMT_Q6_K) {
        dq[1024 + lane * 8 + 2 * j] = (uint8_t)up_lo;
        dq[1024 + lane * 8 + 2 * j + 1] = (uint8_t)up_hi;
      }
    }
  }
}

void launch_pack_kquant(int fmt, const uint8_t* src, int n_out, int k, uint8_t* dst_qs, uint8_t* dst_d,
                        hipStream_t st) {
  const int NR = n_rowgroups(n_out), NQ = n_quads(k);
  const long long total = (long long)NR * 16 * NQ;
  const int blocks = (int)((total + 255) / 256);
  if (fmt == KD_FMT_Q4_K)
    pack_kquant_kernel<KD_FMT_Q4_K><<<blocks, 256, 0, st>>>(src, n_out, k, NR, NQ, dst_qs, dst_d);
  else if (fmt == KD_FMT_Q5_K)
    pack_kquant_kernel<KD_FMT_Q5_K><<<blocks, 256, 0, st>>>(src, n_out, k, NR, NQ, dst_qs, dst_d);
  else
    pack_kquant_kernel<KD_FMT_Q6_K><<<blocks, 256, 0, st>>>(src, n_out, k, NR, NQ, dst_qs, dst_d);
}

template <int RG, int EPI>
void launch_mmvq_kq(int fmt, const MmvqArgs& a, int n_groups, hipStream_t st) {
  if (fmt == KD_FMT_Q4_K)
    launch_mmvq_t<KD_FMT_Q4_K, RG, EPI>(a, n_groups, st);
  else if (fmt == KD_FMT_Q5_K)
    launch_mmvq_t<KD_FMT_Q5_K, RG, EPI>(a, n_groups, st);
  else
    launch_mmvq_t<KD_FMT_Q6_K, RG, EPI>(a, n_groups, st);
}

template void launch_mmvq_kq<kPlainRG, EPI_PLAIN>(int, const MmvqArgs&, int, hipStream_t);
template void launch_mmvq_kq<4, EPI_SWIGLU>(int, const MmvqArgs&, int, hipStream_t);
template void launch_mmvq_kq<2, EPI_RESNORM>(int, const MmvqArgs&, int, hipStream_t);
template void launch_mmvq_kq<1, EPI_ROPE>(int, const MmvqArgs&, int, hipStream_t);

}  // namespace kd
