// Ragged split-K decode attention over per-row fp16 KV caches, and the fp16 KV append.
//
// What is computed (memra-engine 0.72.0, src/decode_batch.rs, ``decode_batch_layers`` phase
// B: one launch over all rows plus one combine, each row reading its own cache through the
// per-row pointer table; hf2q ADR-040 §0.7 F5, batched varlen decode attention with a
// per-query base pointer and kv length): for row b and query head h with KV head
// g = h / (H/G), out = softmax(q . K[0:t_b] * scale) V[0:t_b].
//
// How: keys of row b are cut into S_b chunks of c_b = max(128, ceil(t_b / 256)) keys — a
// function of the row's own t_b only, never of B or of the other rows (the reading of the
// page's rule that every row must run the program of its isolated run).  One workgroup per
// (row, chunk, KV head) reads that head's contiguous K/V stream once for all H/G query heads
// of the group and writes (m, l, o): the chunk's score max, exp-sum and un-normalised
// output.  The combine merges chunks in chunk order: M = max m_s, out = sum e^(m_s-M) o_s /
// sum e^(m_s-M) l_s.  All reductions use fixed trees, so a row's bytes equal its 1-row call.
#include <algorithm>

#include <mutex>

#include "kd_internal.h"

namespace kd {

constexpr int kKvAux = 2;  // cache policy of the K/V loads: non-temporal (each key is read once)

constexpr int kFaMinChunk = 128;
constexpr int kFaMaxSplits = 256;
constexpr int kFaMaxKeys = 128 * 1024;  // t_kv limit: chunk <= 1024 keys

int fa_chunk_for(int t) {
  const int c = ceil_div(t, kFaMaxSplits);
  return c > kFaMinChunk ? c : kFaMinChunk;
}

bool fa_make_plan(FaPlan& p, int B, int H, int G, int hd, const int32_t* t_kv, int forced_chunk) {
  p.B = B;
  p.H = H;
  p.G = G;
  p.hd = hd;
  p.split_off[0] = 0;
  for (int b = 0; b < B; ++b) {
    const int t = t_kv[b];
    const int c = forced_chunk > 0 ? forced_chunk : fa_chunk_for(t);
    p.chunk[b] = c;
    p.t_kv[b] = t;
    p.split_off[b + 1] = p.split_off[b] + ceil_div(t, c);
  }
  for (int b = B; b < KD_MAX_B; ++b) {
    p.chunk[b] = 1;
    p.t_kv[b] = 0;
    p.split_off[b + 1] = p.split_off[B];
  }
  p.n_items = p.split_off[B];
  return true;
}

// Partials: o [items][H][hd] fp32, then m (base-2 scaled) and l [items][H] fp32.
size_t fa_workspace_bytes(const FaPlan& p) {
  return (size_t)p.n_items * p.H * (p.hd + 2) * sizeof(float);
}


// 2^x by the hardware instruction (about 1 ulp; results below 2^-126 flush to zero, which
// only drops probabilities that cannot change an fp32 sum holding a term of 1).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------------
// Split kernel on the matrix cores: 8 waves, each taking 16 keys of every 128-key tile.
//   scores  S^T[key][head] = K[key][:] . q'[head][:] with v_mfma_f32_16x16x32_f16: the A
//           operand is 16 keys x 32 dims of K (lane: key l%16, 8 dims), B is q' (lane: head
//           l%16, the same 8 dims); q' = q * scale * log2(e) * 2^e_h is split into two fp16
//           halves hi + lo (two products), so the scores keep ~22 bits (K is fp16 already).
//           The power of two 2^e_h brings head h's largest |q'| just under 2^14, so the low
//           half stays a normal fp16 number; the products are scaled back by 2^-e_h (exact).
//   output  O[head][dim] += P[head][key] V[key][dim] with v_mfma_f32_16x16x16_f16: A is P
//           (lane: head l%16, keys 4(l/16) .. +3 -- the lane's own score tile entries), B is V
//           (lane: dim 8(l%16) + m of the same 4 keys; one product per m = 0..7); P' = 2^14 p
//           (p <= 1) is split into fp16 hi + lo the same way and the sum scaled back by 2^-14.
// Head slots past R are zero rows of q' and their outputs are dropped.
// ---------------------------------------------------------------------------------------
typedef _Float16 fa_v8h __attribute__((ext_vector_type(8)));
typedef _Float16 fa_v4h __attribute__((ext_vector_type(4)));
typedef float fa_v4f __attribute__((ext_vector_type(4)));
constexpr int kFaWaves = 8;
constexpr int kFaGroupCols = 8;  // query columns of a workgroup whose rows share a cache pass

__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

// FP8 E4M3 caches: two codes (bits 0..7 and 16..23 of c) to two fp16 values, exactly.  The
// code's magnitude bits moved to fp16 bits 13..7 read as an fp16 number equal to the code's
// value times 2^-8 (the exponent biases differ by 8; subnormal codes land on fp16 subnormals),
// so one multiply by 256 gives the value; every E4M3 value is an fp16 number.  The NaN codes,
// which the append never writes for finite inputs, read as 480.
typedef _Float16 fa_v2h __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t c) {
  const uint32_t h = ((c & 0x007F007Fu) << 7) | ((c & 0x00800080u) << 8);
  const fa_v2h v = __builtin_bit_cast(fa_v2h, h) * (fa_v2h){(_Float16)256.0f, (_Float16)256.0f};
  return __builtin_bit_cast(uint32_t, v);
}
// Eight codes (in memory order) to eight fp16 values (in the same order).
__device__ __forceinline__ int4 e4m3x8_to_f16x8(uint2 c) {
  int4 r;
  r.x = (int)e4m3x2_to_f16x2((c.x & 0xFFu) | ((c.x & 0xFF00u) << 8));
  r.y = (int)e4m3x2_to_f16x2(((c.x >> 16) & 0xFFu) | ((c.x >> 8) & 0xFF0000u));
  r.z = (int)e4m3x2_to_f16x2((c.y & 0xFFu) | ((c.y & 0xFF00u) << 8));
  r.w = (int)e4m3x2_to_f16x2(((c.y >> 16) & 0xFFu) | ((c.y >> 8) & 0xFF0000u));
  return r;
}

// Eight int8 codes (in memory order) to eight fp16 values, exactly (|code| <= 127).
__device__ __forceinline__ fa_v8h i8x8_to_f16x8(uint2 c) {
  fa_v8h r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (_Float16)(float)(int8_t)(((e < 4 ? c.x : c.y) >> (8 * (e & 3))) & 0xFF);
  return r;
}
// fp16 number j (0..3) of four packed in a uint2, as fp32.
__device__ __forceinline__ float half_at(uint2 v, int j) {
  const uint32_t w = j < 2 ? v.x : v.y;
  return __half2float(__ushort_as_half((unsigned short)((j & 1) ? (w >> 16) : (w & 0xFFFF))));
}

// MULTI: chunks may span several 128-key tiles (rows longer than 128 x 128 keys).  Without
// it the tile loop runs once, so the running output is not live across a tile's loads and
// the kernel needs fewer registers (more workgroups per CU); the operations are the same.
// C: query columns of the workgroup (R heads of each of the group's rows), C <= 16 -- the
// MFMA's 16 columns.  Column h is head g R + h % R of the group's row h / R; each column
// masks the keys at or past its own row's t_kv, so a row's partials are those of its own
// pass (the keys it does not attend score -inf and weigh exactly 0).
// KF (kd_kv_format): KD_KV_F16 fp16 caches; KD_KV_FP8_E4M3: the caches hold E4M3 codes, each
// lane loads 8 codes where it loads 8 fp16 values otherwise and widens them exactly, so every
// product sees the same operands; KD_KV_Q8_0: int8 rows (Q8_0 blocks of 32 along the head row,
// one fp16 scale each, rows of HD + 16 bytes).  For int8 rows the score product runs on the
// codes (exact in fp16) with one accumulator per 32-dim slice -- one block -- and each key's
// slice sums are scaled by its block scales in fp32, in slice order; the values are the codes
// times their block scale (exact in fp32), split into fp16 hi + lo like p, and the output
// product is issued for p_hi v_hi, p_lo v_hi and p_hi v_lo.
template <int R, int HD, bool MULTI, int C, int KF>
__global__ __launch_bounds__(64 * kFaWaves) void fa_split_kernel(FaPlan p, const float* __restrict__ q,
                                                                          int ldq, RowCaches rc, int capacity,
                                                                          float scale, float* __restrict__ ws) {
  constexpr int NW = kFaWaves;
  constexpr int NC = HD / 32;      // 32-dim slices of the score product
  constexpr int TK = 16 * NW;      // keys per tile
  constexpr float kPScale = 16384.0f, kPInv = 1.0f / 16384.0f;
  static_assert(R <= C && C <= 16, "query columns");
  constexpr bool GROUPED = C > R;  // rows sharing a cache pass; otherwise one row per workgroup
  int item = blockIdx.x;
  const int g = blockIdx.y;
  const int H = p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, gq = lane >> 4;
  const float scale2 = scale * 1.44269504088896341f;
  int b = 0, nrow = 1, sc = 0, k0 = 0, k1 = 0;
  const void* kbase;
  const void* vbase;
  if constexpr (GROUPED) {
    int gi = 0;
#pragma unroll
    for (int i = 1; i < KD_MAX_B; ++i)
      if (item >= p.grp_off[i]) gi = i;
    b = p.grp_row[gi];
    nrow = p.grp_n[gi];
    sc = item - p.grp_off[gi];  // chunk index, the same for every row of the group
    k0 = sc * p.grp_chunk[gi];
    k1 = min(k0 + p.grp_chunk[gi], p.grp_t[gi]);
    kbase = p.grp_k[gi];
    vbase = p.grp_v[gi];
  } else if (gridDim.z > 1) {
    // (chunk, KV head, row) grid: the row is known without reading the plan, so every value
    // the chunk needs comes in one round of loads; chunks past the row's last exit
    b = blockIdx.z;
    sc = blockIdx.x;
    if (sc >= p.split_off[b + 1] - p.split_off[b]) return;
    item = p.split_off[b] + sc;
    k0 = sc * p.chunk[b];
    k1 = min(k0 + p.chunk[b], p.t_kv[b]);
    kbase = rc.k[b];
    vbase = rc.v[b];
  } else {
#pragma unroll
    for (int i = 1; i < KD_MAX_B; ++i)
      if (item >= p.split_off[i]) b = i;
    sc = item - p.split_off[b];
    k0 = sc * p.chunk[b];
    k1 = min(k0 + p.chunk[b], p.t_kv[b]);
    kbase = rc.k[b];
    vbase = rc.v[b];
  }
  const int ncol = GROUPED ? nrow * R : R;
  const int nk = k1 - k0;
  // Grouped: per-column facts, fetched before the K/V loads (loads complete in issue order):
  // the row of column n and, for the columns this thread writes out, their row's t_kv and
  // first split item.
  constexpr int KO = (C * HD + 64 * NW - 1) / (64 * NW);
  int tn = 0, t_out[KO], so_out[KO], t_ml = 0, so_ml = 0;
  if constexpr (GROUPED) {
    tn = p.t_kv[b + (n < ncol ? n / R : 0)];
#pragma unroll
    for (int k = 0; k < KO; ++k) {
      const int h = min((tid + 64 * NW * k) / HD, ncol - 1);
      t_out[k] = p.t_kv[b + h / R];
      so_out[k] = p.split_off[b + h / R];
    }
    const int hm = tid < ncol ? tid : 0;
    t_ml = p.t_kv[b + hm / R];
    so_ml = p.split_off[b + hm / R];
  }

  __shared__ float tmax[2][NW][16];
  __shared__ float red_l[NW][16];
  __shared__ float red_o[NW][C][HD];
  __shared__ __attribute__((aligned(16))) _Float16 qlds[2][NC][16][32];
  __shared__ float qun[16];
  __shared__ float alpha_s[2][16];

  constexpr bool F8 = KF == KD_KV_FP8_E4M3;
  constexpr bool Q8 = KF == KD_KV_Q8_0;
  constexpr uint32_t ES = KF == KD_KV_F16 ? 2 : 1;  // bytes per cache element
  constexpr uint32_t RS = kv_row_bytes(KF, HD);      // bytes per cached key (one head)
  const char* Kg = static_cast<const char*>(kbase) + (size_t)g * capacity * RS;
  const char* Vg = static_cast<const char*>(vbase) + (size_t)g * capacity * RS;
  // descriptors end at key k1: keys past the chunk read zeros, so offsets are base + constants
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg, (uint32_t)k1 * RS);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg, (uint32_t)k1 * RS);

  // q of the heads this wave stages (w, w + 8), fetched before any K/V load so that waiting
  // for it never waits for the tile's K/V bytes (loads complete in issue order)
  float xs[16 / NW][HD / 64];
#pragma unroll
  for (int hs = 0; hs < 16 / NW; ++hs) {
    const int h = w + NW * hs;
#pragma unroll
    for (int i = 0; i < HD / 64; ++i)
      xs[hs][i] = h < ncol ? q[(size_t)(b + h / R) * ldq + (size_t)(g * R + h % R) * HD + lane + 64 * i] : 0.0f;
  }

  // keys of this chunk that column n's row attends (grouped: columns past the group's, and
  // rows that end before this chunk, whose partials are dropped, keep the chunk's count)
  int nkc = nk;
  if constexpr (GROUPED) {
    const int kc = n < ncol ? min(k1, tn) : k1;
    nkc = kc > k0 ? kc - k0 : nk;
  }
  float m_run = -INFINITY;  // running max of head n (every lane of column n holds it)
  float l_run = 0.0f;       // this lane's share of head n's exp-sum
  fa_v4f o[8];              // o[m][s]: head 4gq + s, dim 8n + m (scaled by 2^14)
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] = fa_v4f{0.0f, 0.0f, 0.0f, 0.0f};

  for (int t0 = 0, par = 0; t0 < (MULTI ? nk : 1); t0 += TK, par ^= 1) {
    const int wk = t0 + 16 * w;  // this wave's first key within the chunk
    // K: slice j -> key wk + n, dims 32j + 8gq (8 elements)
    const uint32_t kb = (uint32_t)(k0 + wk + n) * RS + 8 * gq * ES;
    int4 kr[NC];
    uint2 k8[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      if constexpr (F8 || Q8)
        k8[j] = buf8<kKvAux>(rk, kb + j * 32);
      else
        kr[j] = buf16<kKvAux>(rk, kb + j * 64);
    }
    // int8 rows: the block scales of the keys this lane's scores belong to (wk + 4gq + s)
    uint2 ksc[4];
    if constexpr (Q8) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) ksc[s2] = buf8<kKvAux>(rk, (uint32_t)(k0 + wk + 4 * gq + s2) * RS + HD);
    }
    // V: key wk + 4gq + t, dims 8n .. 8n+7 (lanes with 8n >= HD read bytes whose outputs are dropped)
    const uint32_t vb0 = (uint32_t)(k0 + wk + 4 * gq) * RS + 8 * n * ES;
    int4 vr[4];
    uint2 v8[4];
    uint32_t vsc[4];  // int8 rows: the scale pair holding block (8n)/32 of key wk + 4gq + t
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (F8 || Q8)
        v8[t] = buf8<kKvAux>(rv, vb0 + t * RS);
      else
        vr[t] = buf16<kKvAux>(rv, vb0 + t * RS);
      if constexpr (Q8)
        vsc[t] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
            rv, (uint32_t)(k0 + wk + 4 * gq + t) * RS + HD + 4 * (n / 8), 0, kKvAux);
    }
    __builtin_amdgcn_sched_barrier(0);  // every K and V load of the tile ahead of the math
    if (t0 == 0) {
      // q' = q * scale * log2(e) * 2^e_h for the 16 head slots (zero past R), as fp16 hi + lo
      // in LDS in the operand layout [hi/lo][slice][head][32 dims]; wave w stages heads w, w + 8
#pragma unroll
      for (int hs = 0; hs < 16 / NW; ++hs) {
        const int h = w + NW * hs;
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < HD / 64; ++i) {
          xs[hs][i] *= scale2;
          am = fmaxf(am, fabsf(xs[hs][i]));
        }
        am = wave_max(am);
        int ex = 0;
        if (am > 0.0f) frexpf(am, &ex);  // am < 2^ex
        ex = 14 - max(ex, -100);           // |q' 2^ex| < 2^14
#pragma unroll
        for (int i = 0; i < HD / 64; ++i) {
          const int d = lane + 64 * i;
          _Float16 hi, lo;
          split_f16(ldexpf(xs[hs][i], ex), hi, lo);
          qlds[0][d / 32][h][d % 32] = hi;
          qlds[1][d / 32][h][d % 32] = lo;
        }
        if (lane == 0) qun[h] = ldexpf(1.0f, -ex);
      }
      __syncthreads();
    }

    // scores of keys wk + 4gq + s, head n (base 2)
    fa_v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (Q8) {
      // one accumulator per slice (= block), then the keys' block scales in slice order
      fa_v4f accj[NC];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const fa_v8h kv = i8x8_to_f16x8(k8[j]);
        accj[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, *reinterpret_cast<const fa_v8h*>(&qlds[0][j][n][8 * gq]),
                                                         fa_v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        accj[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, *reinterpret_cast<const fa_v8h*>(&qlds[1][j][n][8 * gq]),
                                                         accj[j], 0, 0, 0);
      }
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        float v = half_at(ksc[s2], 0) * accj[0][s2];
#pragma unroll
        for (int j = 1; j < NC; ++j) v = fmaf(half_at(ksc[s2], j), accj[j][s2], v);
        acc[s2] = v;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const fa_v8h kv = __builtin_bit_cast(fa_v8h, F8 ? e4m3x8_to_f16x8(k8[j]) : kr[j]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, *reinterpret_cast<const fa_v8h*>(&qlds[0][j][n][8 * gq]), acc,
                                                     0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, *reinterpret_cast<const fa_v8h*>(&qlds[1][j][n][8 * gq]), acc,
                                                     0, 0, 0);
      }
    }
    const float qunscale = qun[n];
    float pv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      pv[s] = wk + 4 * gq + s < nkc ? acc[s] * qunscale : -INFINITY;
      mx = fmaxf(mx, pv[s]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (gq == 0) tmax[par][w][n] = mx;
    __syncthreads();
    float M = tmax[par][0][n];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, tmax[par][ww][n]);
    const float mnew = fmaxf(m_run, M);
    const float alpha = fast_exp2(m_run - mnew);  // 0 on the first tile
    m_run = mnew;
    l_run *= alpha;
    if (w == 0 && gq == 0) alpha_s[par][n] = alpha;
    fa_v4h ph, pl;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float pe = fast_exp2(pv[s] - mnew);
      l_run += pe;
      _Float16 hi, lo;
      split_f16(pe * kPScale, hi, lo);
      ph[s] = hi;
      pl[s] = lo;
    }
    if (t0 > 0) {  // rescale the running output rows (head 4gq + s) by their heads' alpha
      __syncthreads();
      float al[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) al[s] = alpha_s[par][4 * gq + s];
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int s = 0; s < 4; ++s) o[m][s] *= al[s];
    }
    // O += P V, one product per dim offset m of the lane's 8 dims
    if constexpr (F8) {
#pragma unroll
      for (int t = 0; t < 4; ++t) vr[t] = e4m3x8_to_f16x8(v8[t]);
    }
    if constexpr (Q8) {
      // values = codes times their block scale (exact in fp32), as fp16 hi + lo
      float dv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) dv[t] = __half2float(__ushort_as_half((unsigned short)(((n / 4) & 1) ? (vsc[t] >> 16) : (vsc[t] & 0xFFFF))));
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        fa_v4h vh, vl;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float x = dv[t] * (float)(int8_t)((m < 4 ? (v8[t].x >> (8 * m)) : (v8[t].y >> (8 * (m - 4)))) & 0xFF);
          _Float16 hi, lo;
          split_f16(x, hi, lo);
          vh[t] = hi;
          vl[t] = lo;
        }
        o[m] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vh, o[m], 0, 0, 0);
        o[m] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vh, o[m], 0, 0, 0);
        o[m] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vl, o[m], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        fa_v4h vb;
#pragma unroll
        for (int t = 0; t < 4; ++t) vb[t] = __builtin_bit_cast(fa_v8h, vr[t])[m];
        o[m] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vb, o[m], 0, 0, 0);
        o[m] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vb, o[m], 0, 0, 0);
      }
    }
  }

  // exp-sums: the 4 key groups of the wave, then the waves in order
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (gq == 0) red_l[w][n] = l_run;
  // outputs: this lane holds heads 4gq + s, dims 8n + m
  if (8 * n < HD) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int h = 4 * gq + s;
      if (h < C)
#pragma unroll
        for (int m = 0; m < 8; ++m) red_o[w][h][8 * n + m] = o[m][s];
    }
  }
  __syncthreads();
  float* po = ws;                                  // [items][H][HD]
  float* pm = ws + (size_t)p.n_items * H * HD;     // [items][H]
  float* pl2 = pm + (size_t)p.n_items * H;         // [items][H]
  // column h's partials go to its row's own split item (rows whose keys end before this chunk
  // have no such item: their columns are dropped)
  if constexpr (GROUPED) {
#pragma unroll
    for (int k = 0; k < KO; ++k) {
      const int idx = tid + 64 * NW * k;
      const int h = idx / HD, d = idx % HD;
      if (idx < ncol * HD && k0 < t_out[k]) {
        float v = red_o[0][h][d];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) v += red_o[ww][h][d];
        po[((size_t)(so_out[k] + sc) * H + g * R + h % R) * HD + d] = v * kPInv;
      }
    }
    if (tid < ncol && k0 < t_ml) {
      float l = red_l[0][tid];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) l += red_l[ww][tid];
      const size_t it = (size_t)(so_ml + sc) * H + g * R + tid % R;
      pm[it] = m_run;  // lane tid holds column tid's running max
      pl2[it] = l;
    }
  } else {
    for (int idx = tid; idx < R * HD; idx += 64 * NW) {
      const int h = idx / HD, d = idx % HD;
      float v = red_o[0][h][d];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) v += red_o[ww][h][d];
      po[((size_t)item * H + g * R) * HD + idx] = v * kPInv;
    }
    if (tid < R) {
      float l = red_l[0][tid];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) l += red_l[ww][tid];
      pm[(size_t)item * H + g * R + tid] = m_run;  // lane tid holds head tid's running max
      pl2[(size_t)item * H + g * R + tid] = l;
    }
  }
}

// grid (H, B); HD threads.  Merge the row's chunks in chunk order; optionally quantise.
// Every load of the first FAST chunks -- their m and l, and this thread's dimension of their
// partial outputs -- is issued at once, so a row with up to FAST chunks costs one memory
// round trip; further chunks are merged in LDS-staged batches.  FAST (16, 32, 48 or 64: the
// smallest covering the launch's longest row) only sets how many loads are issued up front:
// the merge runs the same operations in the same order for any FAST.
constexpr int kCombineFast = 64;
constexpr int kCombineStage = 1024;
template <int HD, bool GATED, int FAST>
__global__ __launch_bounds__(HD) void fa_combine_kernel(FaPlan p, const float* __restrict__ ws, float* __restrict__ out,
                                                        int8_t* __restrict__ oq, float* __restrict__ od,
                                                        const float* __restrict__ gate, int ldg) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  // output gate of this element (gated layers), fetched with the partials
  float gv = 0.0f;
  if (GATED) gv = gate[(size_t)b * ldg + (size_t)h * HD + d];
  const int H = p.H;
  const float* po = ws;
  const float* pm = ws + (size_t)p.n_items * H * HD;
  const float* pl = pm + (size_t)p.n_items * H;
  const int s0 = p.split_off[b], S = p.split_off[b + 1] - s0;
  // descriptors over this row's chunks only: chunk s >= S reads zeros
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(po + (size_t)s0 * H * HD, (uint32_t)S * H * HD * 4);
  const __amdgpu_buffer_rsrc_t rm = make_rsrc(pm + (size_t)s0 * H, (uint32_t)S * H * 4);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(pl + (size_t)s0 * H, (uint32_t)S * H * 4);
  const float mv = buf4f(rm, d < S ? (uint32_t)(d * H + h) * 4 : kOOB);  // thread d: chunk d
  const float lv = buf4f(rl, d < S ? (uint32_t)(d * H + h) * 4 : kOOB);
  float ov[FAST];
#pragma unroll
  for (int i = 0; i < FAST; ++i) ov[i] = buf4f(ro, (uint32_t)((i * H + h) * HD + d) * 4);
  __builtin_amdgcn_sched_barrier(0);

  __shared__ float wm[kCombineStage];
  __shared__ float wl[kCombineStage];
  __shared__ float red[HD / 64];
  float M = d < S ? mv : -INFINITY;
  for (int s = d + HD; s < S; s += HD) M = fmaxf(M, pm[(size_t)(s0 + s) * H + h]);
  M = wave_max(M);
  if ((d & 63) == 0) red[d >> 6] = M;
  __syncthreads();
  M = red[0];
  for (int i = 1; i < HD / 64; ++i) M = fmaxf(M, red[i]);
  if (d < S && d < FAST) {
    const float w = fast_exp2(mv - M);
    wm[d] = w;
    wl[d] = w * lv;
  }
  __syncthreads();
  float num = 0.0f, den = 0.0f;
  const int nf = S < FAST ? S : FAST;
#pragma unroll
  for (int i = 0; i < FAST; ++i)
    if (i < nf) {
      num = fmaf(wm[i], ov[i], num);
      den += wl[i];
    }
  for (int base = FAST; base < S; base += kCombineStage) {
    const int n = min(kCombineStage, S - base);
    __syncthreads();
    for (int s = d; s < n; s += HD) {
      const size_t it = (size_t)(s0 + base + s) * H + h;
      const float w = fast_exp2(pm[it] - M);
      wm[s] = w;
      wl[s] = w * pl[it];
    }
    __syncthreads();
    int s = 0;
    for (; s + 8 <= n; s += 8) {
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = po[((size_t)(s0 + base + s + i) * H + h) * HD + d];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        num = fmaf(wm[s + i], o[i], num);
        den += wl[s + i];
      }
    }
    for (; s < n; ++s) {
      num = fmaf(wm[s], po[((size_t)(s0 + base + s) * H + h) * HD + d], num);
      den += wl[s];
    }
  }
  float v = num / den;
  if (GATED) v = v * (1.0f / (1.0f + expf(-gv)));
  out[((size_t)b * H + h) * HD + d] = v;
  if (oq) {
    // 8 lanes per 32-element block: lane d holds dims (d/8)*32 + 4(d%8) .. +3 after a shuffle
    // through LDS; HD/32 blocks per head.
    __shared__ float row[HD];
    row[d] = v;
    __syncthreads();
    const int n = H * HD, NQ = n_quads(n), nbp = NQ * 4;
    if (d < (HD / 32) * 8) {
      const int lb = d >> 3, sub = d & 7;
      const float4 x4 = *reinterpret_cast<const float4*>(row + lb * 32 + 4 * sub);
      const int blk = (h * HD) / 32 + lb;
      quant4_lane8(x4, sub, true, oq + ((size_t)b * NQ + (blk >> 2)) * 128 + (blk & 3) * 8, od + (size_t)b * nbp + blk);
    }
    // padded blocks past H*HD (only when H*HD is not a multiple of 128)
    if (h == H - 1 && d < 8) {
      for (int blk = n / 32; blk < nbp; ++blk)
        quant4_lane8(make_float4(0.0f, 0.0f, 0.0f, 0.0f), d, true,
                     oq + ((size_t)b * NQ + (blk >> 2)) * 128 + (blk & 3) * 8, od + (size_t)b * nbp + blk);
    }
  }
}

template <int R, int HD, int C, int F8>
static void launch_fa_c(const FaPlan& p, const float* q, int ldq, const RowCaches& rc, int capacity, float scale,
                        void* ws, hipStream_t st) {
  int cmax = 0;
  for (int b = 0; b < p.B; ++b) cmax = p.chunk[b] > cmax ? p.chunk[b] : cmax;
  // rows not sharing a cache: a (chunk, KV head, row) grid when it wastes at most an eighth of
  // its workgroups on chunks past short rows' ends, else one workgroup per (item, KV head)
  int smax = 0;
  for (int b = 0; b < p.B; ++b) smax = std::max(smax, p.split_off[b + 1] - p.split_off[b]);
  const bool rows3d = C == R && smax * p.B <= p.n_items + p.n_items / 8;
  const dim3 grid(C > R ? p.grp_off[p.n_grp] : rows3d ? smax : p.n_items, p.G, rows3d ? p.B : 1);
  if (cmax > 16 * kFaWaves)
    fa_split_kernel<R, HD, true, C, F8><<<grid, 64 * kFaWaves, 0, st>>>(p, q, ldq, rc, capacity, scale,
                                                                   static_cast<float*>(ws));
  else
    fa_split_kernel<R, HD, false, C, F8><<<grid, 64 * kFaWaves, 0, st>>>(p, q, ldq, rc, capacity, scale,
                                                                    static_cast<float*>(ws));
}

template <int HD, int FAST>
static void launch_combine(const FaPlan& p, const float* ws, float* out, int8_t* oq, float* od, const float* gate,
                           int ldq, hipStream_t st) {
  if (gate)
    fa_combine_kernel<HD, true, FAST><<<dim3(p.H, p.B), HD, 0, st>>>(p, ws, out, oq, od, gate, ldq);
  else
    fa_combine_kernel<HD, false, FAST><<<dim3(p.H, p.B), HD, 0, st>>>(p, ws, out, oq, od, nullptr, 0);
}

template <int R, int HD>
static void launch_fa_t(const FaPlan& p, const float* q, int ldq, const RowCaches& rc, int capacity, float scale,
                        float* out, int8_t* oq, float* od, void* ws, hipStream_t st, const float* gate, int kvf) {
  if (kvf == KD_KV_FP8_E4M3) {
    if (p.max_grp > 1)
      launch_fa_c<R, HD, kFaGroupCols, KD_KV_FP8_E4M3>(p, q, ldq, rc, capacity, scale, ws, st);
    else
      launch_fa_c<R, HD, R, KD_KV_FP8_E4M3>(p, q, ldq, rc, capacity, scale, ws, st);
  } else if (kvf == KD_KV_Q8_0) {
    if (p.max_grp > 1)
      launch_fa_c<R, HD, kFaGroupCols, KD_KV_Q8_0>(p, q, ldq, rc, capacity, scale, ws, st);
    else
      launch_fa_c<R, HD, R, KD_KV_Q8_0>(p, q, ldq, rc, capacity, scale, ws, st);
  } else {
    if (p.max_grp > 1)
      launch_fa_c<R, HD, kFaGroupCols, KD_KV_F16>(p, q, ldq, rc, capacity, scale, ws, st);
    else
      launch_fa_c<R, HD, R, KD_KV_F16>(p, q, ldq, rc, capacity, scale, ws, st);
  }
  int smax = 0;
  for (int b = 0; b < p.B; ++b) smax = std::max(smax, (int)(p.split_off[b + 1] - p.split_off[b]));
  const float* w = static_cast<const float*>(ws);
  if (smax <= 16)
    launch_combine<HD, 16>(p, w, out, oq, od, gate, ldq, st);
  else if (smax <= 32)
    launch_combine<HD, 32>(p, w, out, oq, od, gate, ldq, st);
  else if (smax <= 48)
    launch_combine<HD, 48>(p, w, out, oq, od, gate, ldq, st);
  else
    launch_combine<HD, kCombineFast>(p, w, out, oq, od, gate, ldq, st);
}

// Rows that can share one pass over their keys: consecutive rows of one cache (same K and V
// base) with the same chunk size, non-decreasing t_kv, and at most kFaGroupCols query columns.
static void fa_group_rows(FaPlan& p, const RowCaches& rc) {
  const int R = p.H / p.G;
  const int cap = R < kFaGroupCols ? kFaGroupCols / R : 1;
  p.n_grp = 0;
  p.max_grp = 0;
  p.grp_off[0] = 0;
  for (int b = 0; b < p.B; ++b) {
    const int i = p.n_grp - 1;
    const bool join = i >= 0 && p.grp_n[i] < cap && rc.k[b] == rc.k[b - 1] && rc.v[b] == rc.v[b - 1] &&
                      p.chunk[b] == p.chunk[b - 1] && p.t_kv[b] >= p.t_kv[b - 1];
    if (join) {
      ++p.grp_n[i];
    } else {
      p.grp_row[p.n_grp] = b;
      p.grp_n[p.n_grp] = 1;
      ++p.n_grp;
    }
  }
  for (int i = 0; i < p.n_grp; ++i) {
    const int first = p.grp_row[i], last = first + p.grp_n[i] - 1;  // the longest row: its chunks cover the group's
    p.grp_off[i + 1] = p.grp_off[i] + (p.split_off[last + 1] - p.split_off[last]);
    p.max_grp = p.grp_n[i] > p.max_grp ? p.grp_n[i] : p.max_grp;
    p.grp_chunk[i] = p.chunk[first];
    p.grp_t[i] = p.t_kv[last];
    p.grp_k[i] = rc.k[first];
    p.grp_v[i] = rc.v[first];
  }
  for (int i = p.n_grp; i < KD_MAX_B; ++i) p.grp_off[i + 1] = p.grp_off[p.n_grp];
}

void launch_fa(const FaPlan& plan, const float* q, int ldq, const RowCaches& rc, int capacity, float scale, float* out,
               int8_t* out_qs, float* out_d, void* ws, hipStream_t st, const float* gate, int kv_fmt) {
  FaPlan p = plan;
  fa_group_rows(p, rc);
  const int R = p.H / p.G;
#define KD_FA_CASE(RR, HH) \
  if (R == RR && p.hd == HH) return launch_fa_t<RR, HH>(p, q, ldq, rc, capacity, scale, out, out_qs, out_d, ws, st, gate, kv_fmt);
  KD_FA_CASE(1, 64) KD_FA_CASE(2, 64) KD_FA_CASE(4, 64) KD_FA_CASE(8, 64)
  KD_FA_CASE(1, 128) KD_FA_CASE(2, 128) KD_FA_CASE(4, 128) KD_FA_CASE(8, 128)
#undef KD_FA_CASE
}

bool fa_shape_supported(int H, int G, int hd) {
  if (G <= 0 || H % G) return false;
  const int R = H / G;
  return (R == 1 || R == 2 || R == 4 || R == 8) && (hd == 64 || hd == 128);
}

int fa_max_keys() { return kFaMaxKeys; }

}  // namespace kd

using namespace kd;

// ---------------------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------------------
static kd_status fa_check(const char* who, const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                          const void* const* k_base, const void* const* v_base, const int32_t* t_kv, const float* out) {
  KD_REQUIRE(B >= 1 && B <= KD_MAX_B, KD_ERR_UNSUPPORTED, "%s: B=%d outside [1,16]", who, B);
  KD_REQUIRE(H > 0 && G > 0, KD_ERR_INVALID, "%s: H=%d G=%d", who, H, G);
  KD_REQUIRE(fa_shape_supported(H, G, hd), KD_ERR_UNSUPPORTED,
             "%s: H/G must be 1, 2, 4 or 8 and hd 64 or 128 (H=%d G=%d hd=%d)", who, H, G, hd);
  KD_REQUIRE(q && k_base && v_base && t_kv && out, KD_ERR_INVALID, "%s: null pointer", who);
  for (int b = 0; b < B; ++b) {
    KD_REQUIRE(k_base[b] && v_base[b], KD_ERR_INVALID, "%s: null cache pointer for row %d", who, b);
    KD_REQUIRE(t_kv[b] >= 1 && t_kv[b] <= fa_max_keys(), KD_ERR_UNSUPPORTED, "%s: t_kv[%d]=%d outside [1, %d]", who, b,
               t_kv[b], fa_max_keys());
  }
  return KD_OK;
}

// Split-partial storage of kd_fa_decode_ragged_noalloc: one array per GPU the library runs
// on, held until the process ends.  Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kFaScratchBytes = 16u << 20;
static __device__ __align__(256) char scratch[kFaScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static kd_status fa_scratch(const char* who, void** out) {
  int dev = -1;
  KD_REQUIRE(hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices, KD_ERR_HIP,
             "%s: no current device (or more than %d)", who, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    KD_REQUIRE(e == hipSuccess && p, KD_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array: %s", who,
               hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KD_OK;
}

// ws == nullptr with use_scratch: the split partials go to this device's scratch array.
static kd_status fa_run(const char* who, const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                        const void* const* k_base, const void* const* v_base, const int32_t* t_kv, int32_t capacity,
                        float scale, float* out, int32_t chunk, void* ws, size_t ws_bytes, void* stream,
                        int kv_fmt = KD_KV_F16, bool use_scratch = false) {
  kd_status s = fa_check(who, q, B, H, G, hd, k_base, v_base, t_kv, out);
  if (s != KD_OK) return s;
  for (int b = 0; b < B; ++b)
    KD_REQUIRE(t_kv[b] <= capacity, KD_ERR_CAPACITY, "%s: t_kv[%d]=%d exceeds capacity %d", who, b, t_kv[b], capacity);
  FaPlan p;
  fa_make_plan(p, B, H, G, hd, t_kv, chunk);
  for (int b = 0; b < B; ++b)
    KD_REQUIRE(p.chunk[b] <= 1024, KD_ERR_UNSUPPORTED, "%s: chunk of %d keys exceeds 1024", who, p.chunk[b]);
  if (use_scratch) {
    KD_REQUIRE(fa_workspace_bytes(p) <= kFaScratchBytes, KD_ERR_WORKSPACE,
               "%s: the split partials need %zu bytes, more than the %zu-byte scratch array", who,
               fa_workspace_bytes(p), kFaScratchBytes);
    s = fa_scratch(who, &ws);
    if (s != KD_OK) return s;
    ws_bytes = kFaScratchBytes;
  }
  KD_REQUIRE(ws && ws_bytes >= fa_workspace_bytes(p), KD_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes,
             fa_workspace_bytes(p));
  RowCaches rc = {};
  for (int b = 0; b < B; ++b) {
    rc.k[b] = const_cast<void*>(k_base[b]);
    rc.v[b] = const_cast<void*>(v_base[b]);
    rc.pos[b] = t_kv[b] - 1;
  }
  launch_fa(p, q, H * hd, rc, capacity, scale, out, nullptr, nullptr, ws, as_stream(stream), nullptr, kv_fmt);
  return check_launch(who);
}

extern "C" size_t kd_fa_decode_workspace(int32_t B, int32_t H, int32_t hd, const int32_t* t_kv) {
  if (B < 1 || B > KD_MAX_B || H <= 0 || hd <= 0 || !t_kv) return 0;
  for (int b = 0; b < B; ++b)
    if (t_kv[b] < 1) return 0;
  FaPlan p;
  fa_make_plan(p, B, H, 1, hd, t_kv, 0);
  return fa_workspace_bytes(p);
}

extern "C" size_t kd_debug_fa_workspace(int32_t B, int32_t H, int32_t hd, const int32_t* t_kv, int32_t chunk) {
  if (B < 1 || B > KD_MAX_B || H <= 0 || hd <= 0 || !t_kv || chunk < 1) return 0;
  for (int b = 0; b < B; ++b)
    if (t_kv[b] < 1) return 0;
  FaPlan p;
  fa_make_plan(p, B, H, 1, hd, t_kv, chunk);
  return fa_workspace_bytes(p);
}

extern "C" kd_status kd_fa_decode_ragged_noalloc(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                                 const void* const* k_base, const void* const* v_base,
                                                 const int32_t* t_kv, int32_t capacity, float scale, float* out,
                                                 void* stream) {
  return fa_run("kd_fa_decode_ragged_noalloc", q, B, H, G, hd, k_base, v_base, t_kv, capacity, scale, out, 0, nullptr,
                0, stream, KD_KV_F16, true);
}

extern "C" kd_status kd_fa_decode_ragged(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                         const void* const* k_base, const void* const* v_base, const int32_t* t_kv,
                                         int32_t capacity, float scale, float* out, void* ws, size_t ws_bytes,
                                         void* stream) {
  return fa_run("kd_fa_decode_ragged", q, B, H, G, hd, k_base, v_base, t_kv, capacity, scale, out, 0, ws, ws_bytes,
                stream);
}

extern "C" kd_status kd_fa_decode_ragged_fp8(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                             const void* const* k_base, const void* const* v_base,
                                             const int32_t* t_kv, int32_t capacity, float scale, float* out, void* ws,
                                             size_t ws_bytes, void* stream) {
  return fa_run("kd_fa_decode_ragged_fp8", q, B, H, G, hd, k_base, v_base, t_kv, capacity, scale, out, 0, ws,
                ws_bytes, stream, KD_KV_FP8_E4M3);
}

extern "C" kd_status kd_fa_decode_ragged_q8(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                            const void* const* k_base, const void* const* v_base, const int32_t* t_kv,
                                            int32_t capacity, float scale, float* out, void* ws, size_t ws_bytes,
                                            void* stream) {
  return fa_run("kd_fa_decode_ragged_q8", q, B, H, G, hd, k_base, v_base, t_kv, capacity, scale, out, 0, ws,
                ws_bytes, stream, KD_KV_Q8_0);
}

extern "C" kd_status kd_debug_fa_decode_chunked(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                                const void* const* k_base, const void* const* v_base,
                                                const int32_t* t_kv, int32_t capacity, float scale, float* out,
                                                int32_t chunk, void* ws, size_t ws_bytes, void* stream) {
  KD_REQUIRE(chunk >= 1, KD_ERR_INVALID, "kd_debug_fa_decode_chunked: chunk=%d", chunk);
  return fa_run("kd_debug_fa_decode_chunked", q, B, H, G, hd, k_base, v_base, t_kv, capacity, scale, out, chunk, ws,
                ws_bytes, stream);
}

static kd_status kv_append_run(const char* who, const float* k, const float* v, int32_t B, int32_t G, int32_t hd,
                               void* const* k_base, void* const* v_base, const int32_t* pos, int32_t capacity,
                               void* stream, int kv_fmt) {
  KD_REQUIRE(B >= 1 && B <= KD_MAX_B, KD_ERR_UNSUPPORTED, "%s: B=%d outside [1,16]", who, B);
  KD_REQUIRE(G > 0 && hd > 0, KD_ERR_INVALID, "%s: G=%d hd=%d", who, G, hd);
  KD_REQUIRE(hd == 64 || hd == 128, KD_ERR_UNSUPPORTED, "%s: hd=%d not 64 or 128", who, hd);
  KD_REQUIRE(k && v && k_base && v_base && pos, KD_ERR_INVALID, "%s: null pointer", who);
  RowCaches rc = {};
  for (int b = 0; b < B; ++b) {
    KD_REQUIRE(k_base[b] && v_base[b], KD_ERR_INVALID, "%s: null cache pointer for row %d", who, b);
    KD_REQUIRE(pos[b] >= 0, KD_ERR_INVALID, "%s: pos[%d]=%d < 0", who, b, pos[b]);
    KD_REQUIRE(pos[b] + 1 <= capacity, KD_ERR_CAPACITY, "%s: pos[%d]=%d does not fit capacity %d", who, b, pos[b],
               capacity);
    for (int a = 0; a < b; ++a)
      KD_REQUIRE(!(k_base[a] == k_base[b] && pos[a] == pos[b]), KD_ERR_INVALID,
                 "%s: rows %d and %d write the same cache slot", who, a, b);
    rc.k[b] = k_base[b];
    rc.v[b] = v_base[b];
    rc.pos[b] = pos[b];
  }
  launch_kv_append(k, v, B, G, hd, rc, capacity, as_stream(stream), kv_fmt);
  return check_launch(who);
}

extern "C" kd_status kd_kv_append(const float* k, const float* v, int32_t B, int32_t G, int32_t hd,
                                  void* const* k_base, void* const* v_base, const int32_t* pos, int32_t capacity,
                                  void* stream) {
  return kv_append_run("kd_kv_append", k, v, B, G, hd, k_base, v_base, pos, capacity, stream, KD_KV_F16);
}

extern "C" kd_status kd_kv_append_fp8(const float* k, const float* v, int32_t B, int32_t G, int32_t hd,
                                      void* const* k_base, void* const* v_base, const int32_t* pos,
                                      int32_t capacity, void* stream) {
  return kv_append_run("kd_kv_append_fp8", k, v, B, G, hd, k_base, v_base, pos, capacity, stream, KD_KV_FP8_E4M3);
}

extern "C" kd_status kd_kv_append_q8(const float* k, const float* v, int32_t B, int32_t G, int32_t hd,
                                     void* const* k_base, void* const* v_base, const int32_t* pos, int32_t capacity,
                                     void* stream) {
  return kv_append_run("kd_kv_append_q8", k, v, B, G, hd, k_base, v_base, pos, capacity, stream, KD_KV_Q8_0);
}
