// Ragged split-K decode attention over per-row fp16 KV caches, and the fp16 KV append.
//
// What is computed (memra-engine 0.72.0, src/decode_batch.rs, ``decode_batch_layers`` phase
// B: one launch over all rows plus one combine, each row reading its own cache through the
// per-row pointer table; hf2q ADR-040 §0.7 F5, batched varlen decode attention with a
// per-query base pointer and kv length): for row b and query head h with KV head
// g = h / (H/G), out = softmax(q . K[0:t_b] * scale) V[0:t_b].
//
// How: keys of row b are cut into S_b chunks of c_b = max(128, ceil(t_b / 128)) keys — a
// function of the row's own t_b only, never of B or of the other rows (the reading of the
// page's rule that every row must run the program of its isolated run).  One workgroup per
// (row, chunk, KV head) reads that head's contiguous K/V stream once for all H/G query heads
// of the group and writes (m, l, o): the chunk's score max, exp-sum and un-normalised
// output.  The combine merges chunks in chunk order: M = max m_s, out = sum e^(m_s-M) o_s /
// sum e^(m_s-M) l_s.  All reductions use fixed trees, so a row's bytes equal its 1-row call.
#include "kd_internal.h"

namespace kd {

#ifndef KD_FA_TK
#define KD_FA_TK 128      // keys per tile when R <= 4
#endif
#ifndef KD_FA_AUX
#define KD_FA_AUX 2       // cache policy of the K/V loads (2: non-temporal)
#endif
#ifndef KD_FA_MIN_WAVES
#define KD_FA_MIN_WAVES 1  // occupancy floor handed to the register allocator (waves per SIMD)
#endif

constexpr int kFaThreads = 256;
constexpr int kFaMinChunk = 128;
constexpr int kFaMaxSplits = 128;
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

__device__ inline void half8_to_float(const int4 u, float* f) {
  const __half2* h = reinterpret_cast<const __half2*>(&u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 t = __half22float2(h[i]);
    f[2 * i] = t.x;
    f[2 * i + 1] = t.y;
  }
}

// 2^x by the hardware instruction (about 1 ulp; results below 2^-126 flush to zero, which
// only drops probabilities that cannot change an fp32 sum holding a term of 1).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of N = 8 or 16 lanes; every lane of the group ends with the
// same bits (each step adds two equal partial sums, in one order or the other).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror: lane i of 8 takes lane 7-i
  if (N == 16) v += dpp_f<0x140>(v);  // row_mirror: lane i of 16 takes lane 15-i
  return v;
}

// Lane geometry of one workgroup (4 waves) over a tile of keys: a key's HD fp16 values are
// read by LPK lanes, 16 bytes (8 dims) each, so one wave load covers KPW whole keys and the
// workgroup SLOTS keys; a tile of TK keys is NL loads per lane for K and NL for V, all
// issued before the first score is computed.
template <int R, int HD>
struct FaShape {
  static constexpr int LPK = HD / 8;
  static constexpr int KPW = 64 / LPK;
  static constexpr int SLOTS = 4 * KPW;
  static constexpr int TK = R <= 4 ? KD_FA_TK : KD_FA_TK / 2;
  static constexpr int NL = TK / SLOTS;
};

// grid (n_items, G); 256 threads.  One workgroup per (row b, split s, KV head g): it reads
// keys [s*c_b, min((s+1)*c_b, t_b)) of head g once for the R query heads of the group, tile
// by tile with a running max (the tile order and every reduction tree are fixed by c_b and
// t_b), and writes the split's partials (m, l, o) for those R heads.
template <int R, int HD>
__global__ __launch_bounds__(kFaThreads, KD_FA_MIN_WAVES) void fa_split_kernel(FaPlan p, const float* __restrict__ q, int ldq,
                                                              RowCaches rc, int capacity, float scale,
                                                              float* __restrict__ ws) {
  using S = FaShape<R, HD>;
  constexpr int LPK = S::LPK, SLOTS = S::SLOTS, TK = S::TK, NL = S::NL;
  constexpr int NOUT = R * HD;  // outputs of one (row, KV head)
  const int item = blockIdx.x, g = blockIdx.y;
  int b = 0;
#pragma unroll
  for (int i = 1; i < KD_MAX_B; ++i)
    if (item >= p.split_off[i]) b = i;
  const int s0 = p.split_off[b];
  const int c = p.chunk[b];
  const int k0 = (item - s0) * c;
  const int k1 = min(k0 + c, p.t_kv[b]);
  const int nk = k1 - k0;
  const int H = p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // scores are carried in base 2: s2 = (q . k) * scale * log2(e), so e^(s - m) = 2^(s2 - m2)
  const float scale2 = scale * 1.44269504088896341f;
  const int dl = lane % LPK;                     // this lane's dims [8 dl, 8 dl + 8)
  const int slot = w * S::KPW + lane / LPK;      // this lane's key slot

  __shared__ float tmax[2][4][R];
  __shared__ float red_l[4][R];
  __shared__ float red_o[4][R][HD];

  float qv[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float4* qr = reinterpret_cast<const float4*>(q + (size_t)b * ldq + (size_t)(g * R + r) * HD + dl * 8);
    const float4 a = qr[0], e = qr[1];
    qv[r][0] = a.x; qv[r][1] = a.y; qv[r][2] = a.z; qv[r][3] = a.w;
    qv[r][4] = e.x; qv[r][5] = e.y; qv[r][6] = e.z; qv[r][7] = e.w;
  }
  // descriptors over keys [0, k1) of head g: loads past the chunk read zeros
  const __half* Kg = static_cast<const __half*>(rc.k[b]) + (size_t)g * capacity * HD;
  const __half* Vg = static_cast<const __half*>(rc.v[b]) + (size_t)g * capacity * HD;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg, (uint32_t)k1 * HD * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg, (uint32_t)k1 * HD * 2);

  float m_run[R], l_acc[R], o_acc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m_run[r] = -INFINITY;
    l_acc[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o_acc[r][e] = 0.0f;
  }

  for (int t0 = 0, par = 0; t0 < nk; t0 += TK, par ^= 1) {
    const int nt = min(TK, nk - t0);
    int4 kr[NL], vr[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int j = i * SLOTS + slot;
      const uint32_t off = j < nt ? ((uint32_t)(k0 + t0 + j) * HD + dl * 8) * 2 : kOOB;
      kr[i] = buf16<KD_FA_AUX>(rk, off);
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int j = i * SLOTS + slot;
      const uint32_t off = j < nt ? ((uint32_t)(k0 + t0 + j) * HD + dl * 8) * 2 : kOOB;
      vr[i] = buf16<KD_FA_AUX>(rv, off);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every K and V load of the tile ahead of the math
    // scores of this lane's NL keys for the R heads (identical in the LPK lanes of a key)
    float sc[R][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float kf[8];
      half8_to_float(kr[i], kf);
      const bool live = i * SLOTS + slot < nt;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(qv[r][e], kf[e], part);
        part = group_sum<LPK>(part);
        sc[r][i] = live ? part * scale2 : -INFINITY;
      }
    }
    // tile max per head: lane keys, then the key groups of the wave, then the 4 waves
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float mx = sc[r][0];
#pragma unroll
      for (int i = 1; i < NL; ++i) mx = fmaxf(mx, sc[r][i]);
#pragma unroll
      for (int m = LPK; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
      if (lane == 0) tmax[par][w][r] = mx;
    }
    __syncthreads();
    float alpha[R], mnew[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float M = fmaxf(fmaxf(tmax[par][0][r], tmax[par][1][r]), fmaxf(tmax[par][2][r], tmax[par][3][r]));
      mnew[r] = fmaxf(m_run[r], M);
      alpha[r] = fast_exp2(m_run[r] - mnew[r]);  // 0 on the first tile
      m_run[r] = mnew[r];
      l_acc[r] *= alpha[r];
#pragma unroll
      for (int e = 0; e < 8; ++e) o_acc[r][e] *= alpha[r];
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float vf[8];
      half8_to_float(vr[i], vf);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float pj = fast_exp2(sc[r][i] - mnew[r]);
        l_acc[r] += pj;
#pragma unroll
        for (int e = 0; e < 8; ++e) o_acc[r][e] = fmaf(pj, vf[e], o_acc[r][e]);
      }
    }
  }

  // key groups of the wave (butterfly), then the 4 waves through LDS in wave order
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int m = LPK; m < 64; m <<= 1) {
      l_acc[r] += __shfl_xor(l_acc[r], m, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) o_acc[r][e] += __shfl_xor(o_acc[r][e], m, 64);
    }
  }
  if (lane < LPK) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[w][r][dl * 8 + e] = o_acc[r][e];
      if (dl == 0) red_l[w][r] = l_acc[r];
    }
  }
  __syncthreads();

  float* po = ws;                                  // [items][H][HD]
  float* pm = ws + (size_t)p.n_items * H * HD;     // [items][H]
  float* pl = pm + (size_t)p.n_items * H;          // [items][H]
  for (int idx = tid; idx < NOUT; idx += kFaThreads) {
    const int r = idx / HD, d = idx % HD;
    po[((size_t)item * H + g * R) * HD + idx] =
        ((red_o[0][r][d] + red_o[1][r][d]) + red_o[2][r][d]) + red_o[3][r][d];
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (tid == r) {
      pm[(size_t)item * H + g * R + r] = m_run[r];
      pl[(size_t)item * H + g * R + r] = ((red_l[0][r] + red_l[1][r]) + red_l[2][r]) + red_l[3][r];
    }
}

// grid (H, B); HD threads.  Merge the row's chunks in chunk order; optionally quantise.
// The chunk maxima and their weights e^(m_s - M) are staged in LDS once; each thread then
// reads its dimension of every chunk's partial with 8 loads in flight at a time.
constexpr int kCombineStage = 1024;
template <int HD>
__global__ __launch_bounds__(HD) void fa_combine_kernel(FaPlan p, const float* __restrict__ ws, float* __restrict__ out,
                                                        int8_t* __restrict__ oq, float* __restrict__ od) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int H = p.H;
  const float* po = ws;
  const float* pm = ws + (size_t)p.n_items * H * HD;
  const float* pl = pm + (size_t)p.n_items * H;
  const int s0 = p.split_off[b], S = p.split_off[b + 1] - s0;
  __shared__ float wm[kCombineStage];
  __shared__ float wl[kCombineStage];
  __shared__ float red[HD / 64];
  float M = -INFINITY;
  for (int s = d; s < S; s += HD) M = fmaxf(M, pm[(size_t)(s0 + s) * H + h]);
  M = wave_max(M);
  if ((d & 63) == 0) red[d >> 6] = M;
  __syncthreads();
  M = red[0];
  for (int i = 1; i < HD / 64; ++i) M = fmaxf(M, red[i]);
  float num = 0.0f, den = 0.0f;
  for (int base = 0; base < S; base += kCombineStage) {
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
  const float v = num / den;
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

template <int R, int HD>
static void launch_fa_t(const FaPlan& p, const float* q, int ldq, const RowCaches& rc, int capacity, float scale,
                        float* out, int8_t* oq, float* od, void* ws, hipStream_t st) {
  fa_split_kernel<R, HD><<<dim3(p.n_items, p.G), kFaThreads, 0, st>>>(p, q, ldq, rc, capacity, scale,
                                                                      static_cast<float*>(ws));
  fa_combine_kernel<HD><<<dim3(p.H, p.B), HD, 0, st>>>(p, static_cast<const float*>(ws), out, oq, od);
}

void launch_fa(const FaPlan& p, const float* q, int ldq, const RowCaches& rc, int capacity, float scale, float* out,
               int8_t* out_qs, float* out_d, void* ws, hipStream_t st) {
  const int R = p.H / p.G;
#define KD_FA_CASE(RR, HH) \
  if (R == RR && p.hd == HH) return launch_fa_t<RR, HH>(p, q, ldq, rc, capacity, scale, out, out_qs, out_d, ws, st);
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

static kd_status fa_run(const char* who, const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                        const void* const* k_base, const void* const* v_base, const int32_t* t_kv, int32_t capacity,
                        float scale, float* out, int32_t chunk, void* ws, size_t ws_bytes, void* stream) {
  kd_status s = fa_check(who, q, B, H, G, hd, k_base, v_base, t_kv, out);
  if (s != KD_OK) return s;
  for (int b = 0; b < B; ++b)
    KD_REQUIRE(t_kv[b] <= capacity, KD_ERR_CAPACITY, "%s: t_kv[%d]=%d exceeds capacity %d", who, b, t_kv[b], capacity);
  FaPlan p;
  fa_make_plan(p, B, H, G, hd, t_kv, chunk);
  for (int b = 0; b < B; ++b)
    KD_REQUIRE(p.chunk[b] <= 1024, KD_ERR_UNSUPPORTED, "%s: chunk of %d keys exceeds 1024", who, p.chunk[b]);
  KD_REQUIRE(ws && ws_bytes >= fa_workspace_bytes(p), KD_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes,
             fa_workspace_bytes(p));
  RowCaches rc = {};
  for (int b = 0; b < B; ++b) {
    rc.k[b] = const_cast<void*>(k_base[b]);
    rc.v[b] = const_cast<void*>(v_base[b]);
    rc.pos[b] = t_kv[b] - 1;
  }
  launch_fa(p, q, H * hd, rc, capacity, scale, out, nullptr, nullptr, ws, as_stream(stream));
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

extern "C" kd_status kd_fa_decode_ragged(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                         const void* const* k_base, const void* const* v_base, const int32_t* t_kv,
                                         int32_t capacity, float scale, float* out, void* ws, size_t ws_bytes,
                                         void* stream) {
  return fa_run("kd_fa_decode_ragged", q, B, H, G, hd, k_base, v_base, t_kv, capacity, scale, out, 0, ws, ws_bytes,
                stream);
}

extern "C" kd_status kd_debug_fa_decode_chunked(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                                const void* const* k_base, const void* const* v_base,
                                                const int32_t* t_kv, int32_t capacity, float scale, float* out,
                                                int32_t chunk, void* ws, size_t ws_bytes, void* stream) {
  KD_REQUIRE(chunk >= 1, KD_ERR_INVALID, "kd_debug_fa_decode_chunked: chunk=%d", chunk);
  return fa_run("kd_debug_fa_decode_chunked", q, B, H, G, hd, k_base, v_base, t_kv, capacity, scale, out, chunk, ws,
                ws_bytes, stream);
}

extern "C" kd_status kd_kv_append(const float* k, const float* v, int32_t B, int32_t G, int32_t hd,
                                  void* const* k_base, void* const* v_base, const int32_t* pos, int32_t capacity,
                                  void* stream) {
  KD_REQUIRE(B >= 1 && B <= KD_MAX_B, KD_ERR_UNSUPPORTED, "kd_kv_append: B=%d outside [1,16]", B);
  KD_REQUIRE(G > 0 && hd > 0, KD_ERR_INVALID, "kd_kv_append: G=%d hd=%d", G, hd);
  KD_REQUIRE(hd == 64 || hd == 128, KD_ERR_UNSUPPORTED, "kd_kv_append: hd=%d not 64 or 128", hd);
  KD_REQUIRE(k && v && k_base && v_base && pos, KD_ERR_INVALID, "kd_kv_append: null pointer");
  RowCaches rc = {};
  for (int b = 0; b < B; ++b) {
    KD_REQUIRE(k_base[b] && v_base[b], KD_ERR_INVALID, "kd_kv_append: null cache pointer for row %d", b);
    KD_REQUIRE(pos[b] >= 0, KD_ERR_INVALID, "kd_kv_append: pos[%d]=%d < 0", b, pos[b]);
    KD_REQUIRE(pos[b] + 1 <= capacity, KD_ERR_CAPACITY, "kd_kv_append: pos[%d]=%d does not fit capacity %d", b, pos[b],
               capacity);
    for (int a = 0; a < b; ++a)
      KD_REQUIRE(!(k_base[a] == k_base[b] && pos[a] == pos[b]), KD_ERR_INVALID,
                 "kd_kv_append: rows %d and %d write the same cache slot", a, b);
    rc.k[b] = k_base[b];
    rc.v[b] = v_base[b];
    rc.pos[b] = pos[b];
  }
  launch_kv_append(k, v, B, G, hd, rc, capacity, as_stream(stream));
  return check_launch("kd_kv_append");
}
