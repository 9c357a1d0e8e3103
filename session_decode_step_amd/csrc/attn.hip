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

// Partials: o [items][H][hd] fp32, then m and l [items][H] fp32.
size_t fa_workspace_bytes(const FaPlan& p) {
  return (size_t)p.n_items * p.H * (p.hd + 2) * sizeof(float);
}

__device__ inline void half8_to_float(const uint4 u, float* f) {
  const __half2* h = reinterpret_cast<const __half2*>(&u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 t = __half22float2(h[i]);
    f[2 * i] = t.x;
    f[2 * i + 1] = t.y;
  }
}

// grid (n_items, G); 256 threads.  R = query heads per KV head; HD = head dim.
template <int R, int HD>
__global__ __launch_bounds__(kFaThreads) void fa_split_kernel(FaPlan p, const float* __restrict__ q, int ldq,
                                                              RowCaches rc, int capacity, float scale,
                                                              float* __restrict__ ws) {
  constexpr int DPL = HD / 8;   // dims per lane in the score phase (8 lanes per key)
  constexpr int DV = HD / 16;   // dims per lane in the PV phase (16 lanes per key row)
  extern __shared__ float smem[];
  const int item = blockIdx.x, g = blockIdx.y;
  // row of this item
  int b = 0;
#pragma unroll
  for (int i = 1; i < KD_MAX_B; ++i)
    if (item >= p.split_off[i]) b = i;
  const int s = item - p.split_off[b];
  const int c = p.chunk[b];
  const int k0 = s * c;
  const int k1 = min(k0 + c, p.t_kv[b]);
  const int nk = k1 - k0;
  const int H = p.H;
  float* sc = smem;                      // [R][c] scores, then probabilities
  float* red = smem + R * c;             // [4][R][HD]
  __shared__ float ml[R][2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const __half* Kg = static_cast<const __half*>(rc.k[b]) + (size_t)g * capacity * HD;
  const __half* Vg = static_cast<const __half*>(rc.v[b]) + (size_t)g * capacity * HD;

  // ---- phase 1: scores.  32 groups of 8 lanes; a group owns one key at a time.
  {
    const int grp = tid >> 3, sub = tid & 7;
    float qv[R][DPL];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float* qr = q + (size_t)b * ldq + (size_t)(g * R + r) * HD + sub * DPL;
#pragma unroll
      for (int i = 0; i < DPL; ++i) qv[r][i] = qr[i];
    }
    for (int j = grp; j < nk; j += 32) {
      const __half* kp = Kg + (size_t)(k0 + j) * HD + sub * DPL;
      float kf[DPL];
#pragma unroll
      for (int i = 0; i < DPL; i += 8) half8_to_float(*reinterpret_cast<const uint4*>(kp + i), kf + i);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) part = fmaf(qv[r][i], kf[i], part);
        part += __shfl_xor(part, 1, 64);
        part += __shfl_xor(part, 2, 64);
        part += __shfl_xor(part, 4, 64);
        if (sub == 0) sc[r * c + j] = part * scale;
      }
    }
  }
  __syncthreads();

  // ---- phase 2: per-head max and exp-sum over the chunk (wave r % 4 owns head r).
  for (int r = w; r < R; r += 4) {
    float m = -INFINITY;
    for (int j = lane; j < nk; j += 64) m = fmaxf(m, sc[r * c + j]);
    m = wave_max(m);
    float l = 0.0f;
    for (int j = lane; j < nk; j += 64) {
      const float e = expf(sc[r * c + j] - m);
      sc[r * c + j] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      ml[r][0] = m;
      ml[r][1] = l;
    }
  }
  __syncthreads();

  // ---- phase 3: o[r][:] = sum_j p[r][j] V[j][:].  16 key slots (4 per wave), 16 lanes per row.
  {
    const int kg = lane >> 4, dl = lane & 15;
    const int slot = w * 4 + kg;
    float o[R][DV];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < DV; ++i) o[r][i] = 0.0f;
    for (int j = slot; j < nk; j += 16) {
      const __half* vp = Vg + (size_t)(k0 + j) * HD + dl * DV;
      float vf[DV];
      if (DV == 8) {
        half8_to_float(*reinterpret_cast<const uint4*>(vp), vf);
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(vp);
        const __half2* h2 = reinterpret_cast<const __half2*>(&u);
#pragma unroll
        for (int i = 0; i < DV / 2; ++i) {
          const float2 t = __half22float2(h2[i]);
          vf[2 * i] = t.x;
          vf[2 * i + 1] = t.y;
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float pj = sc[r * c + j];
#pragma unroll
        for (int i = 0; i < DV; ++i) o[r][i] = fmaf(pj, vf[i], o[r][i]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < DV; ++i) {
        float v = o[r][i];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        o[r][i] = v;
      }
    if (kg == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < DV; ++i) red[(w * R + r) * HD + dl * DV + i] = o[r][i];
    }
  }
  __syncthreads();
  float* po = ws;                                    // [items][H][HD]
  float* pm = ws + (size_t)p.n_items * H * HD;       // [items][H]
  float* pl = pm + (size_t)p.n_items * H;            // [items][H]
  for (int t = tid; t < R * HD; t += kFaThreads) {
    const int r = t / HD, d = t % HD;
    const float v = ((red[(0 * R + r) * HD + d] + red[(1 * R + r) * HD + d]) + red[(2 * R + r) * HD + d]) +
                    red[(3 * R + r) * HD + d];
    po[((size_t)item * H + g * R + r) * HD + d] = v;
  }
  if (tid < R) {
    pm[(size_t)item * H + g * R + tid] = ml[tid][0];
    pl[(size_t)item * H + g * R + tid] = ml[tid][1];
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
      const float w = expf(pm[it] - M);
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
  int cmax = 1;
  for (int b = 0; b < p.B; ++b) cmax = p.chunk[b] > cmax ? p.chunk[b] : cmax;
  const size_t shm = (size_t)(R * cmax + 4 * R * HD) * sizeof(float);
  fa_split_kernel<R, HD><<<dim3(p.n_items, p.G), kFaThreads, shm, st>>>(p, q, ldq, rc, capacity, scale,
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
