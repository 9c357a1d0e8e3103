// Row-parallel operations of the batched decode step: RMSNorm (optionally fused with the
// residual add and with the activation quantiser), NEOX RoPE with per-row positions fused
// with the fp16 KV append, SwiGLU fused with the quantiser, and the residual add.
//
// These are the row ops that "batch trivially" on the memra-engine page (src/decode_batch.rs
// module header) and that hf2q ADR-040 batches as single dispatches over N rows (§0.12,
// batched norm / RoPE / KV-encode).  Every kernel processes each row independently with a
// reduction order fixed by the row length, so row b's result never depends on B.
#include "kd_internal.h"

namespace kd {

// ---------------------------------------------------------------------------------------
// RMSNorm (+ residual add) (+ quantise).  One 256-thread workgroup per row.
// ---------------------------------------------------------------------------------------
// Thread layout: 8 lanes per 32-element block (lane sub holds 4 consecutive elements as a
// float4), 32 blocks per pass of the 256 threads; the row stays in registers between the
// sum of squares and the normalise + quantise pass.  Sum of squares: per thread in pass
// order, then a fixed xor tree per wave, then the 4 wave sums in wave order.
template <int MAXP>
__global__ __launch_bounds__(256) void norm_quant_kernel(const float* __restrict__ x, const float* __restrict__ r,
                                                         const float* __restrict__ g, int n, float eps,
                                                         float* __restrict__ x1_out, float* __restrict__ y_out,
                                                         int8_t* __restrict__ qs, float* __restrict__ qd) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, sub = tid & 7, lb = tid >> 3;
  const int nb = n / 32, NQ = n_quads(n), nbp = NQ * 4;
  const int P = ceil_div(nbp, 32);
  const float* xr = x + (size_t)b * n;
  const float* rr = r ? r + (size_t)b * n : nullptr;
  float4 v[MAXP], gg[MAXP];
  float ss = 0.0f;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {  // x, r and the gains are all fetched before the reduction
    v[p] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    gg[p] = v[p];
    const int blk = p * 32 + lb;
    if (p < P && blk < nb) {
      const int c = blk * 32 + 4 * sub;
      v[p] = *reinterpret_cast<const float4*>(xr + c);
      gg[p] = *reinterpret_cast<const float4*>(g + c);
      if (rr) v[p] = f4_add(v[p], *reinterpret_cast<const float4*>(rr + c));
    }
    ss = fmaf(v[p].x, v[p].x, ss);
    ss = fmaf(v[p].y, v[p].y, ss);
    ss = fmaf(v[p].z, v[p].z, ss);
    ss = fmaf(v[p].w, v[p].w, ss);
  }
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)n + eps);
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const int blk = p * 32 + lb;
    float4 y = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (p < P && blk < nb) {
      const int c = blk * 32 + 4 * sub;
      y = make_float4((v[p].x * inv) * gg[p].x, (v[p].y * inv) * gg[p].y, (v[p].z * inv) * gg[p].z,
                      (v[p].w * inv) * gg[p].w);
      if (x1_out) *reinterpret_cast<float4*>(x1_out + (size_t)b * n + c) = v[p];
      if (y_out) *reinterpret_cast<float4*>(y_out + (size_t)b * n + c) = y;
    }
    if (qs && p < P)
      quant4_lane8(y, sub, blk < nbp, qs + ((size_t)b * NQ + (blk >> 2)) * 128 + (blk & 3) * 8,
                   qd + (size_t)b * nbp + blk);
  }
}

int norm_max_len() { return 16 * 1024; }

void launch_norm_quant(const float* x, const float* r, const float* g, int B, int n, float eps, float* x1_out,
                       float* y_out, int8_t* qs, float* d, hipStream_t st) {
  const int P = ceil_div(n_quads(n) * 4, 32);
  if (P <= 4)
    norm_quant_kernel<4><<<B, 256, 0, st>>>(x, r, g, n, eps, x1_out, y_out, qs, d);
  else if (P <= 8)
    norm_quant_kernel<8><<<B, 256, 0, st>>>(x, r, g, n, eps, x1_out, y_out, qs, d);
  else
    norm_quant_kernel<16><<<B, 256, 0, st>>>(x, r, g, n, eps, x1_out, y_out, qs, d);
}

// ---------------------------------------------------------------------------------------
// RoPE tables and RoPE + KV append
// ---------------------------------------------------------------------------------------
__global__ void rope_table_kernel(RowCaches rc, int B, int hd, double base, float* __restrict__ cs) {
  const int half = hd / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * half) return;
  const int b = idx / half, i = idx % half;
  const float2 v = rope_cs(rc.pos[b], i, hd, base);
  cs[2 * idx] = v.x;
  cs[2 * idx + 1] = v.y;
}

void launch_rope_table(const RowCaches& rc, int B, int hd, float base, float* cs, hipStream_t st) {
  const int total = B * hd / 2;
  rope_table_kernel<<<ceil_div(total, 256), 256, 0, st>>>(rc, B, hd, (double)base, cs);
}

// int8 cache rows (Q8_0 blocks along the head row): thread i of a block of hd/2 threads holds
// elements i and i + hd/2 of one (head, position) row, so the 32-element block of each lies in
// its half of the threads (lanes 0..31 or 32..63 of the wave).  Per block a = max |x|, the
// stored scale d = fp16(a / 127), codes round-half-away(x / d) clamped to [-127, 127] (0 when
// d is 0); codes at bytes [0, hd) of the row, scales at [hd, hd + hd/16).  Every thread of the
// block must call it (the maxima are 32-lane shuffles).
__device__ __forceinline__ void q8_store_pair(uint8_t* row, int hd, int i, float x0, float x1) {
  const int half = hd / 2;
  float m0 = fabsf(x0), m1 = fabsf(x1);
#pragma unroll
  for (int mask = 16; mask >= 1; mask >>= 1) {
    m0 = fmaxf(m0, __shfl_xor(m0, mask, 32));
    m1 = fmaxf(m1, __shfl_xor(m1, mask, 32));
  }
  const __half d0 = __float2half_rn(m0 / 127.0f), d1 = __float2half_rn(m1 / 127.0f);
  const float f0 = __half2float(d0), f1 = __half2float(d1);
  int c0 = 0, c1 = 0;
  if (f0 != 0.0f) {
    c0 = (int)roundf(x0 / f0);
    c0 = c0 > 127 ? 127 : (c0 < -127 ? -127 : c0);
  }
  if (f1 != 0.0f) {
    c1 = (int)roundf(x1 / f1);
    c1 = c1 > 127 ? 127 : (c1 < -127 ? -127 : c1);
  }
  row[i] = (uint8_t)(int8_t)c0;
  row[i + half] = (uint8_t)(int8_t)c1;
  __half* sc = reinterpret_cast<__half*>(row + hd);
  if ((i & 31) == 0) {
    sc[i / 32] = d0;
    sc[(i + half) / 32] = d1;
  }
}

// grid (H + 2G, B); block hd/2 threads.  Head index h < H: query (rotate in place);
// H <= h < H+G: key (rotate, store fp16); h >= H+G: value (store fp16).  cs is the per-step
// table, or null to evaluate the same fp64 expression inline.
// QK-norm (qn / kn non-null: per-head gains [hd]): each q and k head is RMS-normalised over
// its hd values before the rotation, y = x * (1 / sqrt(sum(x^2) / hd + eps)) * gain, with the
// head's sum of squares added by a fixed butterfly over the block's single wave.
__global__ void rope_append_kernel(float* __restrict__ qkv, int ldqkv, int H, int G, int hd,
                                   const float* __restrict__ cs, double base, RowCaches rc, int capacity,
                                   int append, const float* __restrict__ qn, const float* __restrict__ kn,
                                   float eps) {
  const int h = blockIdx.x, b = blockIdx.y, i = threadIdx.x;
  const int half = hd / 2;
  float* row = qkv + (size_t)b * ldqkv + (size_t)h * hd;
  const int pos = rc.pos[b];
  if (h < H + G) {
    const float2 t = cs ? make_float2(cs[2 * (b * half + i)], cs[2 * (b * half + i) + 1]) : rope_cs(pos, i, hd, base);
    const float c = t.x, s = t.y;
    float x0 = row[i], x1 = row[i + half];
    const float* gn = h < H ? qn : kn;
    if (gn) {  // uniform per block
      float ss = fmaf(x1, x1, x0 * x0);
      for (int m = half / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, half);
      const float inv = 1.0f / sqrtf(ss / (float)hd + eps);
      x0 = x0 * inv * gn[i];
      x1 = x1 * inv * gn[i + half];
    }
    const float y0 = fmaf(x0, c, -(x1 * s));
    const float y1 = fmaf(x0, s, x1 * c);
    row[i] = y0;
    row[i + half] = y1;
    if (h >= H && append == 3) {
      q8_store_pair(static_cast<uint8_t*>(rc.k[b]) + ((size_t)(h - H) * capacity + pos) * kv_q8_row_bytes(hd), hd, i,
                    y0, y1);
    } else if (h >= H && append) {
      const size_t o = ((size_t)(h - H) * capacity + pos) * hd;
      if (append == 2) {
        uint8_t* K = static_cast<uint8_t*>(rc.k[b]) + o;
        K[i] = (uint8_t)f32_to_e4m3(y0);
        K[i + half] = (uint8_t)f32_to_e4m3(y1);
      } else {
        __half* K = static_cast<__half*>(rc.k[b]) + o;
        K[i] = __float2half_rn(y0);
        K[i + half] = __float2half_rn(y1);
      }
    }
  } else if (append == 3) {
    q8_store_pair(static_cast<uint8_t*>(rc.v[b]) + ((size_t)(h - H - G) * capacity + pos) * kv_q8_row_bytes(hd), hd,
                  i, row[i], row[i + half]);
  } else if (append) {
    const size_t o = ((size_t)(h - H - G) * capacity + pos) * hd;
    if (append == 2) {
      uint8_t* V = static_cast<uint8_t*>(rc.v[b]) + o;
      V[i] = (uint8_t)f32_to_e4m3(row[i]);
      V[i + half] = (uint8_t)f32_to_e4m3(row[i + half]);
    } else {
      __half* V = static_cast<__half*>(rc.v[b]) + o;
      V[i] = __float2half_rn(row[i]);
      V[i + half] = __float2half_rn(row[i + half]);
    }
  }
}

void launch_rope_append(float* qkv, int ldqkv, int B, int H, int G, int hd, const float* cs, const RowCaches& rc,
                        int capacity, bool append, hipStream_t st, float base, const float* q_norm,
                        const float* k_norm, float eps, int kv_fmt) {
  dim3 grid(append ? H + 2 * G : H + G, B);
  const int mode = !append ? 0 : kv_fmt == KD_KV_Q8_0 ? 3 : kv_fmt == KD_KV_FP8_E4M3 ? 2 : 1;
  rope_append_kernel<<<grid, hd / 2, 0, st>>>(qkv, ldqkv, H, G, hd, cs, (double)base, rc, capacity, mode, q_norm,
                                              k_norm, eps);
}

// Plain KV append (no rotation): k and v rows [B][G][hd] fp32 -> fp16 (or E4M3 codes) at pos.
template <bool F8>
__global__ void kv_append_kernel(const float* __restrict__ k, const float* __restrict__ v, int G, int hd,
                                 RowCaches rc, int capacity) {
  const int g = blockIdx.x, b = blockIdx.y;
  const size_t src = ((size_t)b * G + g) * hd;
  const size_t o = ((size_t)g * capacity + rc.pos[b]) * hd;
  for (int i = threadIdx.x; i < hd; i += blockDim.x) {
    if (F8) {
      static_cast<uint8_t*>(rc.k[b])[o + i] = (uint8_t)f32_to_e4m3(k[src + i]);
      static_cast<uint8_t*>(rc.v[b])[o + i] = (uint8_t)f32_to_e4m3(v[src + i]);
    } else {
      static_cast<__half*>(rc.k[b])[o + i] = __float2half_rn(k[src + i]);
      static_cast<__half*>(rc.v[b])[o + i] = __float2half_rn(v[src + i]);
    }
  }
}

// int8 rows: grid (G, B), hd/2 threads, thread i codes elements i and i + hd/2 of k and of v.
__global__ void kv_append_q8_kernel(const float* __restrict__ k, const float* __restrict__ v, int G, int hd,
                                    RowCaches rc, int capacity) {
  const int g = blockIdx.x, b = blockIdx.y, i = threadIdx.x, half = hd / 2;
  const size_t src = ((size_t)b * G + g) * hd;
  const size_t o = ((size_t)g * capacity + rc.pos[b]) * kv_q8_row_bytes(hd);
  q8_store_pair(static_cast<uint8_t*>(rc.k[b]) + o, hd, i, k[src + i], k[src + i + half]);
  q8_store_pair(static_cast<uint8_t*>(rc.v[b]) + o, hd, i, v[src + i], v[src + i + half]);
}

void launch_kv_append(const float* k, const float* v, int B, int G, int hd, const RowCaches& rc, int capacity,
                      hipStream_t st, int kv_fmt) {
  if (kv_fmt == KD_KV_Q8_0) {
    kv_append_q8_kernel<<<dim3(G, B), hd / 2, 0, st>>>(k, v, G, hd, rc, capacity);
    return;
  }
  const bool kv_fp8 = kv_fmt == KD_KV_FP8_E4M3;
  if (kv_fp8)
    kv_append_kernel<true><<<dim3(G, B), 64, 0, st>>>(k, v, G, hd, rc, capacity);
  else
    kv_append_kernel<false><<<dim3(G, B), 64, 0, st>>>(k, v, G, hd, rc, capacity);
}

// ---------------------------------------------------------------------------------------
// SwiGLU (+ quantise): grid (ceil(blocks / 32), rows), 8 lanes per 32-element block.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void swiglu_quant_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                           int n, int ld, float* __restrict__ a_out,
                                                           int8_t* __restrict__ qs, float* __restrict__ qd) {
  const int b = blockIdx.y;
  const int sub = threadIdx.x & 7;
  const int blk = blockIdx.x * 32 + (threadIdx.x >> 3);
  const int nb = n / 32, NQ = n_quads(n), nbp = NQ * 4;
  float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (blk < nb) {
    const int c = blk * 32 + 4 * sub;
    const float4 gv = *reinterpret_cast<const float4*>(g + (size_t)b * ld + c);
    const float4 uv = *reinterpret_cast<const float4*>(u + (size_t)b * ld + c);
    a.x = (gv.x / (1.0f + expf(-gv.x))) * uv.x;
    a.y = (gv.y / (1.0f + expf(-gv.y))) * uv.y;
    a.z = (gv.z / (1.0f + expf(-gv.z))) * uv.z;
    a.w = (gv.w / (1.0f + expf(-gv.w))) * uv.w;
    if (a_out) *reinterpret_cast<float4*>(a_out + (size_t)b * n + c) = a;
  }
  if (qs)
    quant4_lane8(a, sub, blk < nbp, qs + ((size_t)b * NQ + (blk >> 2)) * 128 + (blk & 3) * 8, qd + (size_t)b * nbp + blk);
}

void launch_swiglu_quant(const float* g, const float* u, int rows, int n, int ld, float* a_out, int8_t* qs, float* d,
                         hipStream_t st) {
  dim3 grid(ceil_div(n_quads(n) * 4, 32), rows);
  swiglu_quant_kernel<<<grid, 256, 0, st>>>(g, u, n, ld, a_out, qs, d);
}

__global__ void add_kernel(const float* __restrict__ x, const float* __restrict__ y, float* __restrict__ z, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) z[i] = x[i] + y[i];
}

void launch_add(const float* x, const float* y, float* z, size_t n, hipStream_t st) {
  add_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(x, y, z, n);
}

}  // namespace kd

using namespace kd;

// ---------------------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------------------
#define ROWS_OK(who, B, n)                                                                       \
  KD_REQUIRE((B) >= 1 && (B) <= KD_MAX_B, KD_ERR_UNSUPPORTED, "%s: B=%d outside [1,16]", who, (int)(B)); \
  KD_REQUIRE((n) > 0, KD_ERR_INVALID, "%s: n=%d", who, (int)(n))

extern "C" kd_status kd_rmsnorm_rows(const float* x, const float* g, float* y, int32_t B, int32_t n, float eps,
                                     void* stream) {
  ROWS_OK("kd_rmsnorm_rows", B, n);
  KD_REQUIRE(n % 32 == 0 && n <= norm_max_len(), KD_ERR_UNSUPPORTED,
             "kd_rmsnorm_rows: n=%d is not a multiple of 32 in [32, %d]", n, norm_max_len());
  KD_REQUIRE(x && g && y, KD_ERR_INVALID, "kd_rmsnorm_rows: null pointer");
  KD_REQUIRE(aligned16(x) && aligned16(g) && aligned16(y), KD_ERR_INVALID, "kd_rmsnorm_rows: unaligned");
  launch_norm_quant(x, nullptr, g, B, n, eps, nullptr, y, nullptr, nullptr, as_stream(stream));
  return check_launch("kd_rmsnorm_rows");
}

extern "C" kd_status kd_add_rmsnorm_rows(const float* x, const float* r, const float* g, float* x1, float* y,
                                         int32_t B, int32_t n, float eps, void* stream) {
  ROWS_OK("kd_add_rmsnorm_rows", B, n);
  KD_REQUIRE(n % 32 == 0 && n <= norm_max_len(), KD_ERR_UNSUPPORTED,
             "kd_add_rmsnorm_rows: n=%d is not a multiple of 32 in [32, %d]", n, norm_max_len());
  KD_REQUIRE(x && r && g && x1 && y, KD_ERR_INVALID, "kd_add_rmsnorm_rows: null pointer");
  KD_REQUIRE(aligned16(x) && aligned16(r) && aligned16(g) && aligned16(x1) && aligned16(y), KD_ERR_INVALID,
             "kd_add_rmsnorm_rows: unaligned");
  launch_norm_quant(x, r, g, B, n, eps, x1, y, nullptr, nullptr, as_stream(stream));
  return check_launch("kd_add_rmsnorm_rows");
}

extern "C" kd_status kd_rope_neox_rows(float* x, int32_t B, int32_t n_heads, int32_t hd, const int32_t* pos,
                                       float base, void* stream) {
  ROWS_OK("kd_rope_neox_rows", B, n_heads);
  KD_REQUIRE(hd == 64 || hd == 128, KD_ERR_UNSUPPORTED, "kd_rope_neox_rows: hd=%d not 64 or 128", hd);
  KD_REQUIRE(x && pos, KD_ERR_INVALID, "kd_rope_neox_rows: null pointer");
  RowCaches rc = {};
  for (int b = 0; b < B; ++b) {
    KD_REQUIRE(pos[b] >= 0, KD_ERR_INVALID, "kd_rope_neox_rows: pos[%d]=%d < 0", b, pos[b]);
    rc.pos[b] = pos[b];
  }
  // Rotate all n_heads heads of each row in place; cos/sin evaluated inline (no table).
  launch_rope_append(x, n_heads * hd, B, n_heads, 0, hd, nullptr, rc, 0, false, as_stream(stream), base);
  return check_launch("kd_rope_neox_rows");
}

extern "C" kd_status kd_swiglu_rows(const float* g, const float* u, float* a, int32_t B, int32_t n, void* stream) {
  ROWS_OK("kd_swiglu_rows", B, n);
  KD_REQUIRE(n % 32 == 0, KD_ERR_UNSUPPORTED, "kd_swiglu_rows: n=%d is not a multiple of 32", n);
  KD_REQUIRE(g && u && a, KD_ERR_INVALID, "kd_swiglu_rows: null pointer");
  KD_REQUIRE(aligned16(g) && aligned16(u) && aligned16(a), KD_ERR_INVALID, "kd_swiglu_rows: unaligned");
  launch_swiglu_quant(g, u, B, n, n, a, nullptr, nullptr, as_stream(stream));
  return check_launch("kd_swiglu_rows");
}

extern "C" kd_status kd_add_rows(const float* x, const float* y, float* z, int32_t B, int32_t n, void* stream) {
  ROWS_OK("kd_add_rows", B, n);
  KD_REQUIRE(x && y && z, KD_ERR_INVALID, "kd_add_rows: null pointer");
  launch_add(x, y, z, (size_t)B * n, as_stream(stream));
  return check_launch("kd_add_rows");
}
