// One batched decode step over a layer stack (kd_decode_step) and the library plumbing.
//
// Launch sequence per layer (memra-engine 0.72.0, src/decode_batch.rs, ``decode_batch_layers``
// Full-attention arm, without the QK-norm and output-gate variants; hf2q ADR-040 §0.4 and
// §0.7 F2: one [N, hidden] forward per tick with every projection at m = N):
//   [residual add +] attn_norm + quantise        (norm_quant)
//   q/k/v product at m = B                         (mmvq)
//   RoPE with per-row positions + fp16 KV append  (rope_append: phase A, all rows)
//   split-K attention + combine + quantise        (fa: phase B, all rows)
//   o product                                      (mmvq)
//   residual add + post-attention norm + quantise (norm_quant)
//   gate, up products -> silu_mul + quantise -> down product   (dense FFN)
//   or router + expert buckets -> grouped gate/up -> silu_mul -> grouped down,
//      shared expert, rank-ordered combine                       (MoE FFN)
// The residual add that closes a layer is fused into the next layer's norm.  The number of
// launches is independent of B (B is a grid dimension, never a host loop: hf2q ADR-040
// §0.12, the "N as a grid dimension, constant dispatch" plan).  Nothing here synchronises
// the stream or copies host data to the device: per-row positions and cache addresses
// travel as kernel arguments.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "kd_internal.h"

namespace kd {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

kd_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: HIP launch failed: %s", what, hipGetErrorString(e));
    return KD_ERR_HIP;
  }
  return KD_OK;
}

}  // namespace kd

using namespace kd;

struct kd_model {
  kd_model_desc desc;
  std::vector<kd_layer_desc> layers;
  int max_k;       // longest activation row any product reads
  bool linear;     // some layer is a gated delta-rule linear-attention layer
  int ssm_c;       // linear layers: conv channels C = 2 d_state n_k + d_state n_v
  int ssm_vd;      // value dim d_state n_v
  int ssm_nin;     // rows of the input projection: C + d_v + 2 n_v
  size_t ring_floats, state_floats;  // one ring buffer, one state buffer
};

extern "C" const char* kd_last_error(void) { return g_err; }
extern "C" const char* kd_version(void) { return "kd 0.1.0 gfx950 (mfma_i32_16x16x32_i8 mmvq, split-K fa_decode)"; }

// ---------------------------------------------------------------------------------------
// Model
// ---------------------------------------------------------------------------------------
static kd_status check_weight(const char* name, int il, const kd_weight& w, int n_out, int k, bool quant_only = true) {
  KD_REQUIRE(w.qs, KD_ERR_INVALID, "kd_model_create: layer %d %s: null qs", il, name);
  KD_REQUIRE(w.n_out == n_out && w.k == k, KD_ERR_INVALID, "kd_model_create: layer %d %s: shape %d x %d, expected %d x %d",
             il, name, w.n_out, w.k, n_out, k);
  if (quant_only) {
    KD_REQUIRE(w.fmt == KD_FMT_Q8_0 || w.fmt == KD_FMT_Q4_0 || w.fmt == KD_FMT_Q4_K || w.fmt == KD_FMT_Q5_K ||
                   w.fmt == KD_FMT_Q6_K,
               KD_ERR_UNSUPPORTED, "kd_model_create: layer %d %s: format %d is not a quantised weight format", il, name,
               w.fmt);
    KD_REQUIRE(w.d, KD_ERR_INVALID, "kd_model_create: layer %d %s: null scales", il, name);
    KD_REQUIRE(mmvq_fmt_ok(w.fmt, k), KD_ERR_UNSUPPORTED,
               "kd_model_create: layer %d %s: k=%d not a multiple of the format's block (32; K-quants 256)", il, name, k);
    KD_REQUIRE(aligned16(w.qs) && aligned16(w.d), KD_ERR_INVALID, "kd_model_create: layer %d %s: unaligned", il, name);
    KD_REQUIRE(mmvq_weight_fits(w.fmt, n_out, k), KD_ERR_UNSUPPORTED,
               "kd_model_create: layer %d %s: %d x %d exceeds the product's limits (k <= %d, tiled codes under 2 GiB)",
               il, name, n_out, k, mmvq_max_k());
  }
  return KD_OK;
}

#define KD_TRY(expr)                 \
  do {                               \
    const kd_status s_ = (expr);     \
    if (s_ != KD_OK) return s_;      \
  } while (0)

extern "C" kd_status kd_model_create(const kd_model_desc* desc, kd_model** out) {
  KD_REQUIRE(desc && out, KD_ERR_INVALID, "kd_model_create: null argument");
  const kd_model_desc& m = *desc;
  KD_REQUIRE(m.n_layers >= 1 && m.layers, KD_ERR_INVALID, "kd_model_create: n_layers=%d", m.n_layers);
  KD_REQUIRE(m.d > 0 && m.d % 32 == 0 && m.d <= norm_max_len(), KD_ERR_UNSUPPORTED,
             "kd_model_create: d=%d not a multiple of 32 in [32, %d]", m.d, norm_max_len());
  KD_REQUIRE(fa_shape_supported(m.n_head, m.n_head_kv, m.head_dim), KD_ERR_UNSUPPORTED,
             "kd_model_create: H=%d G=%d hd=%d unsupported (H/G in {1,2,4,8}, hd in {64,128})", m.n_head, m.n_head_kv,
             m.head_dim);
  KD_REQUIRE(m.rms_eps > 0 && m.rope_base > 0, KD_ERR_INVALID, "kd_model_create: eps / rope base");
  KD_REQUIRE(m.kv_format == KD_KV_F16 || m.kv_format == KD_KV_FP8_E4M3 || m.kv_format == KD_KV_Q8_0, KD_ERR_INVALID,
             "kd_model_create: kv_format=%d", m.kv_format);
  const int H = m.n_head, G = m.n_head_kv, hd = m.head_dim, d = m.d;
  const bool moe = m.n_experts > 0;
  if (moe) {
    KD_REQUIRE(m.n_experts <= moe_max_experts() && m.n_expert_used >= 1 && m.n_expert_used <= moe_max_topk() &&
                   m.n_expert_used <= m.n_experts,
               KD_ERR_UNSUPPORTED, "kd_model_create: experts %d / used %d", m.n_experts, m.n_expert_used);
    KD_REQUIRE(m.expert_ffn > 0 && m.expert_ffn % 32 == 0 && m.shared_ffn > 0 && m.shared_ffn % 32 == 0 && d % 16 == 0,
               KD_ERR_UNSUPPORTED, "kd_model_create: expert widths must be multiples of 32 (Fe=%d Fs=%d)", m.expert_ffn,
               m.shared_ffn);
    KD_REQUIRE(m.ffn == 0, KD_ERR_INVALID, "kd_model_create: dense ffn and experts both set");
  }
  KD_REQUIRE(m.ffn >= 0 && m.ffn % 32 == 0, KD_ERR_UNSUPPORTED, "kd_model_create: ffn=%d", m.ffn);
  bool any_linear = false;
  for (int il = 0; il < m.n_layers; ++il) any_linear |= m.layers[il].mixer == 1;
  const int ssm_ds = m.ssm_d_state, ssm_nk = m.ssm_n_k, ssm_nv = m.ssm_n_v, ssm_dc = m.ssm_d_conv;
  if (any_linear) {
    KD_REQUIRE(ssm_ds == gdn_state_dim(), KD_ERR_UNSUPPORTED, "kd_model_create: ssm_d_state=%d (only %d)", ssm_ds,
               gdn_state_dim());
    KD_REQUIRE(ssm_nk >= 1 && ssm_nv >= ssm_nk && ssm_nv % ssm_nk == 0 && ssm_nv <= 1024, KD_ERR_UNSUPPORTED,
               "kd_model_create: ssm_n_k=%d ssm_n_v=%d (n_v a multiple of n_k)", ssm_nk, ssm_nv);
    KD_REQUIRE(ssm_dc >= 2 && ssm_dc <= 8, KD_ERR_UNSUPPORTED, "kd_model_create: ssm_d_conv=%d outside [2, 8]", ssm_dc);
  }
  const int ssm_c = 2 * ssm_ds * ssm_nk + ssm_ds * ssm_nv, ssm_vd = ssm_ds * ssm_nv;
  const int ssm_nin = ssm_c + ssm_vd + 2 * ssm_nv;
  for (int il = 0; il < m.n_layers; ++il) {
    const kd_layer_desc& L = m.layers[il];
    KD_REQUIRE(L.attn_norm, KD_ERR_INVALID, "kd_model_create: layer %d: null attn_norm", il);
    KD_REQUIRE(L.mixer == 0 || L.mixer == 1, KD_ERR_INVALID, "kd_model_create: layer %d: mixer=%d", il, L.mixer);
    if (L.mixer == 1) {
      KD_REQUIRE(L.ssm_conv && L.ssm_dt && L.ssm_a && L.ssm_norm, KD_ERR_INVALID,
                 "kd_model_create: layer %d: linear layer without its conv, dt, a or norm arrays", il);
      KD_REQUIRE(aligned16(L.ssm_norm), KD_ERR_INVALID, "kd_model_create: layer %d: ssm_norm must be 16-byte aligned",
                 il);
      KD_REQUIRE(!L.q_norm && !L.k_norm && L.swa_window == 0 && L.attn_gate == 0 && L.wqkv_pair_rows == 0,
                 KD_ERR_INVALID, "kd_model_create: layer %d: attention options set on a linear layer", il);
      KD_TRY(check_weight("wqkv (linear input projection)", il, L.wqkv, ssm_nin, d));
      KD_TRY(check_weight("wo (linear out projection)", il, L.wo, d, ssm_vd));
    }
    KD_REQUIRE(L.swa_window >= 0, KD_ERR_INVALID, "kd_model_create: layer %d: swa_window=%d < 0", il, L.swa_window);
    KD_REQUIRE(!L.q_norm == !L.k_norm, KD_ERR_INVALID, "kd_model_create: layer %d: q_norm and k_norm go together", il);
    KD_REQUIRE(!L.q_norm || L.wqkv_pair_rows == 0, KD_ERR_UNSUPPORTED,
               "kd_model_create: layer %d: QK-norm needs the canonical wqkv layout (wqkv_pair_rows = 0)", il);
    KD_REQUIRE(m.kv_format != KD_KV_Q8_0 || L.wqkv_pair_rows == 0, KD_ERR_UNSUPPORTED,
               "kd_model_create: layer %d: int8 KV caches need the canonical wqkv layout (wqkv_pair_rows = 0)", il);
    KD_REQUIRE(L.attn_gate == 0 || L.attn_gate == 1, KD_ERR_INVALID, "kd_model_create: layer %d: attn_gate=%d", il,
               L.attn_gate);
    if (L.mixer == 0) {
      KD_TRY(check_weight("wqkv", il, L.wqkv, (H + 2 * G + (L.attn_gate ? H : 0)) * hd, d));
      KD_REQUIRE(L.wqkv_pair_rows == 0 || L.wqkv_pair_rows == 1, KD_ERR_INVALID,
                 "kd_model_create: layer %d: wqkv_pair_rows=%d", il, L.wqkv_pair_rows);
      KD_TRY(check_weight("wo", il, L.wo, d, H * hd));
    }
    if (m.ffn > 0 || moe) KD_REQUIRE(L.ffn_norm, KD_ERR_INVALID, "kd_model_create: layer %d: null ffn_norm", il);
    if (m.ffn > 0) {
      if (L.w_up.qs) {
        KD_TRY(check_weight("w_gate", il, L.w_gate, m.ffn, d));
        KD_TRY(check_weight("w_up", il, L.w_up, m.ffn, d));
      } else {
        KD_REQUIRE(mmvq_swiglu_fits(d), KD_ERR_UNSUPPORTED,
                   "kd_model_create: layer %d: d=%d exceeds the fused SwiGLU product's LDS", il, d);
        KD_TRY(check_weight("w_gate (interleaved gate+up)", il, L.w_gate, 2 * m.ffn, d));
        KD_REQUIRE(m.ffn % 32 == 0, KD_ERR_UNSUPPORTED,
                   "kd_model_create: interleaved gate/up needs ffn %% 32 == 0 (ffn=%d)", m.ffn);
      }
      KD_TRY(check_weight("w_down", il, L.w_down, d, m.ffn));
    }
    if (moe) {
      KD_REQUIRE(L.router, KD_ERR_INVALID, "kd_model_create: layer %d: null router", il);
      if (L.e_up.qs) {
        KD_TRY(check_weight("e_gate", il, L.e_gate, m.n_experts * m.expert_ffn, d));
        KD_TRY(check_weight("e_up", il, L.e_up, m.n_experts * m.expert_ffn, d));
      } else {  // each expert's gate and up interleaved in blocks of 32 rows
        KD_REQUIRE(mmvq_swiglu_fits(d), KD_ERR_UNSUPPORTED,
                   "kd_model_create: layer %d: d=%d exceeds the fused SwiGLU product's LDS", il, d);
        KD_TRY(check_weight("e_gate (interleaved expert gate+up)", il, L.e_gate, m.n_experts * 2 * m.expert_ffn, d));
      }
      KD_TRY(check_weight("e_down", il, L.e_down, m.n_experts * d, m.expert_ffn));
      KD_REQUIRE(m.expert_ffn % 16 == 0, KD_ERR_UNSUPPORTED, "kd_model_create: expert_ffn %% 16");
      if (L.s_up.qs) {
        KD_TRY(check_weight("s_gate", il, L.s_gate, m.shared_ffn, d));
        KD_TRY(check_weight("s_up", il, L.s_up, m.shared_ffn, d));
      } else {
        KD_REQUIRE(mmvq_swiglu_fits(d), KD_ERR_UNSUPPORTED,
                   "kd_model_create: layer %d: d=%d exceeds the fused SwiGLU product's LDS", il, d);
        KD_TRY(check_weight("s_gate (interleaved shared gate+up)", il, L.s_gate, 2 * m.shared_ffn, d));
      }
      KD_TRY(check_weight("s_down", il, L.s_down, d, m.shared_ffn));
    }
  }
  if (m.vocab > 0) {
    KD_TRY(check_weight("lm_head", -1, m.lm_head, m.vocab, d));
  }
  kd_model* mm = new (std::nothrow) kd_model;
  KD_REQUIRE(mm, KD_ERR_INVALID, "kd_model_create: out of host memory");
  mm->desc = m;
  mm->layers.assign(m.layers, m.layers + m.n_layers);
  mm->desc.layers = mm->layers.data();
  int mk = d;
  mk = H * hd > mk ? H * hd : mk;
  mk = m.ffn > mk ? m.ffn : mk;
  mk = m.shared_ffn > mk ? m.shared_ffn : mk;
  if (any_linear) mk = ssm_vd > mk ? ssm_vd : mk;
  mm->max_k = mk;
  mm->linear = any_linear;
  mm->ssm_c = any_linear ? ssm_c : 0;
  mm->ssm_vd = any_linear ? ssm_vd : 0;
  mm->ssm_nin = any_linear ? ssm_nin : 0;
  mm->ring_floats = any_linear ? (size_t)(ssm_dc - 1) * ssm_c : 0;
  mm->ring_floats = (mm->ring_floats + 3) & ~(size_t)3;  // each buffer 16-byte aligned
  mm->state_floats = any_linear ? (size_t)ssm_nv * ssm_ds * ssm_ds : 0;
  *out = mm;
  return KD_OK;
}

extern "C" void kd_model_destroy(kd_model* m) { delete m; }

extern "C" size_t kd_recurrent_state_bytes(const kd_model* m) {
  if (!m || !m->linear) return 0;
  return sizeof(float) * 2 * (m->ring_floats + m->state_floats);
}

// ---------------------------------------------------------------------------------------
// Workspace
// ---------------------------------------------------------------------------------------
namespace {
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

struct StepBufs {
  float *xa, *xb, *f, *qkv, *attn, *o, *gu, *z, *cs, *sgu;
  float *lq, *lk, *lv, *lg, *lb, *lo;  // linear layers: prep outputs and the state step's output
  int8_t *act_qs, *act2_qs, *hq_qs, *actn_qs;
  float *act_d, *act2_d, *hq_d, *actn_d, *ss;
  void* fa_ws;
  int32_t *ids, *count, *rows, *pairs;
  float *p, *gup, *yp, *rlog, *shq_d;
  int8_t* shq_qs;
  int8_t* lm_qs;
  float* lm_d;
};

size_t carve_step(const kd_model* m, int B, const FaPlan& plan, void* ws, StepBufs& s) {
  const kd_model_desc& d = m->desc;
  const int H = d.n_head, G = d.n_head_kv, hd = d.head_dim, D = d.d;
  Carve c(ws);
  s.xa = c.take<float>((size_t)B * D);
  s.xb = c.take<float>((size_t)B * D);
  s.f = c.take<float>((size_t)B * D);
  s.o = c.take<float>((size_t)B * D);
  s.z = c.take<float>((size_t)B * D);
  // q, k, v and (gated layers) the gate; linear layers: their input projection's rows
  s.qkv = c.take<float>((size_t)B * std::max((2 * H + 2 * G) * hd, m->ssm_nin));
  if (m->linear) {
    const size_t hv = (size_t)B * d.ssm_n_v;
    s.lq = c.take<float>(hv * d.ssm_d_state);
    s.lk = c.take<float>(hv * d.ssm_d_state);
    s.lv = c.take<float>(hv * d.ssm_d_state);
    s.lo = c.take<float>(hv * d.ssm_d_state);
    s.lg = c.take<float>(hv);
    s.lb = c.take<float>(hv);
  }
  s.attn = c.take<float>((size_t)B * H * hd);
  s.cs = c.take<float>((size_t)B * hd);
  s.act_qs = c.take<int8_t>((size_t)B * n_quads(m->max_k) * 128);
  s.act_d = c.take<float>((size_t)B * n_quads(m->max_k) * 4);
  s.fa_ws = c.take<char>(fa_workspace_bytes(plan));
  s.gu = d.ffn ? c.take<float>((size_t)B * 2 * d.ffn) : nullptr;
  s.act2_qs = d.ffn ? c.take<int8_t>((size_t)B * n_quads(d.ffn) * 128) : nullptr;  // SwiGLU output rows
  s.act2_d = d.ffn ? c.take<float>((size_t)B * n_quads(d.ffn) * 4) : nullptr;
  // FFN input when the O product starts the RMSNorm: Q8 codes of x1 * gain, block sums of x1^2
  s.actn_qs = d.ffn ? c.take<int8_t>((size_t)B * n_quads(D) * 128) : nullptr;
  s.actn_d = d.ffn ? c.take<float>((size_t)B * n_quads(D) * 4) : nullptr;
  s.ss = d.ffn ? c.take<float>((size_t)B * (D / 32)) : nullptr;
  if (d.n_experts) {
    const int K = d.n_expert_used, E = d.n_experts, Fe = d.expert_ffn, Fs = d.shared_ffn;
    s.ids = c.take<int32_t>((size_t)B * K);
    s.p = c.take<float>((size_t)B * K);
    s.rlog = c.take<float>((size_t)B * E);
    s.count = c.take<int32_t>(E);
    s.rows = c.take<int32_t>((size_t)E * 16);
    s.pairs = c.take<int32_t>((size_t)E * 16);
    s.gup = c.take<float>((size_t)B * K * 2 * Fe);
    s.hq_qs = c.take<int8_t>((size_t)B * K * n_quads(Fe) * 128);
    s.hq_d = c.take<float>((size_t)B * K * n_quads(Fe) * 4);
    s.yp = c.take<float>((size_t)B * K * D);
    s.sgu = c.take<float>((size_t)B * 2 * Fs);
    s.shq_qs = c.take<int8_t>((size_t)B * n_quads(Fs) * 128);  // the shared expert's SwiGLU rows
    s.shq_d = c.take<float>((size_t)B * n_quads(Fs) * 4);
  }
  return c.off + 256;
}

bool plan_for(const kd_model* m, int B, const int32_t* pos, FaPlan& plan) {
  int32_t t[KD_MAX_B];
  for (int b = 0; b < B; ++b) t[b] = pos[b] + 1;
  return fa_make_plan(plan, B, m->desc.n_head, m->desc.n_head_kv, m->desc.head_dim, t, 0);
}
}  // namespace

extern "C" size_t kd_decode_step_workspace(const kd_model* m, int32_t B, const int32_t* pos) {
  if (!m || B < 1 || B > KD_MAX_B || !pos) return 0;
  for (int b = 0; b < B; ++b)
    if (pos[b] < 0) return 0;
  FaPlan plan;
  plan_for(m, B, pos, plan);
  StepBufs s;
  return carve_step(m, B, plan, nullptr, s);
}

// ---------------------------------------------------------------------------------------
// The step
// ---------------------------------------------------------------------------------------
namespace {
// Device-to-device copy of n floats (or int32s) for the step record; false on failure.
bool trace_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  if (hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st) != hipSuccess) {
    set_error("kd_debug_decode_step_trace: copy failed");
    return false;
  }
  return true;
}
// Copy the codes of `rows` activation rows of length k (tiled layout) into record slot `slot`
// of a per-layer code array whose rows hold k_slot >= k columns (nothing if the array is not
// requested).
bool trace_codes(int8_t* dst, size_t slot, const int8_t* src, int rows, int k, hipStream_t st, int k_slot = 0) {
  if (!dst) return true;
  k_slot = k_slot > k ? k_slot : k;
  const size_t row = (size_t)n_quads(k) * 128, row_slot = (size_t)n_quads(k_slot) * 128;
  if (hipMemcpy2DAsync(dst + slot * rows * row_slot, row_slot, src, row, row, rows, hipMemcpyDeviceToDevice, st) !=
      hipSuccess) {
    set_error("kd_debug_decode_step_trace: copy failed");
    return false;
  }
  return true;
}
}  // namespace

static kd_status decode_step_impl(const kd_model* m, int32_t B, const float* x_in, const int32_t* pos,
                                  void* const* k_base, void* const* v_base, int32_t capacity, float* out, void* ws,
                                  size_t ws_bytes, const kd_step_trace* tr, void* stream) {
  KD_REQUIRE(m, KD_ERR_INVALID, "kd_decode_step: null model");
  KD_REQUIRE(B >= 1 && B <= KD_MAX_B, KD_ERR_UNSUPPORTED, "kd_decode_step: B=%d outside [1,16]", B);
  KD_REQUIRE(x_in && pos && k_base && v_base && out, KD_ERR_INVALID, "kd_decode_step: null pointer");
  KD_REQUIRE(aligned16(x_in) && aligned16(out), KD_ERR_INVALID, "kd_decode_step: x_in and out must be 16-byte aligned");
  const kd_model_desc& d = m->desc;
  const int L = d.n_layers, H = d.n_head, G = d.n_head_kv, hd = d.head_dim, D = d.d;
  for (int b = 0; b < B; ++b) {
    KD_REQUIRE(pos[b] >= 0, KD_ERR_INVALID, "kd_decode_step: pos[%d]=%d < 0", b, pos[b]);
    KD_REQUIRE(pos[b] + 1 <= capacity, KD_ERR_CAPACITY, "kd_decode_step: pos[%d]=%d does not fit capacity %d", b,
               pos[b], capacity);
    KD_REQUIRE(pos[b] + 1 <= fa_max_keys(), KD_ERR_UNSUPPORTED, "kd_decode_step: pos[%d]=%d beyond %d keys", b, pos[b],
               fa_max_keys());
  }
  for (int il = 0; il < L; ++il)
    for (int b = 0; b < B; ++b) {
      void* kb = k_base[(size_t)il * B + b];
      if (m->layers[il].mixer == 1) {  // a recurrent state per row, never shared
        KD_REQUIRE(kb && aligned16(kb), KD_ERR_INVALID,
                   "kd_decode_step: recurrent state of layer %d row %d null or unaligned", il, b);
        const size_t rb = kd_recurrent_state_bytes(m);
        for (int a = 0; a < b; ++a) {
          const char *pa = static_cast<const char*>(k_base[(size_t)il * B + a]), *pb = static_cast<const char*>(kb);
          KD_REQUIRE(pa + rb <= pb || pb + rb <= pa, KD_ERR_INVALID,
                     "kd_decode_step: rows %d and %d share a recurrent state (layer %d)", a, b, il);
        }
        continue;
      }
      void* vb = v_base[(size_t)il * B + b];
      KD_REQUIRE(kb && vb, KD_ERR_INVALID, "kd_decode_step: null cache pointer (layer %d row %d)", il, b);
      KD_REQUIRE(aligned16(kb) && aligned16(vb), KD_ERR_INVALID, "kd_decode_step: cache (layer %d row %d) unaligned", il,
                 b);
      for (int a = 0; a < b; ++a)
        KD_REQUIRE(!(k_base[(size_t)il * B + a] == kb && pos[a] == pos[b]), KD_ERR_INVALID,
                   "kd_decode_step: rows %d and %d write the same cache slot (layer %d)", a, b, il);
    }
  FaPlan plan;
  plan_for(m, B, pos, plan);
  StepBufs s;
  const size_t need = carve_step(m, B, plan, nullptr, s);
  KD_REQUIRE(ws && ws_bytes >= need, KD_ERR_WORKSPACE, "kd_decode_step: workspace %zu < %zu bytes", ws_bytes, need);
  void* ws_al = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
  KD_REQUIRE(ws_bytes - ((char*)ws_al - (char*)ws) >= need - 256, KD_ERR_WORKSPACE, "kd_decode_step: workspace alignment");
  carve_step(m, B, plan, ws_al, s);

  hipStream_t st = as_stream(stream);
  const bool moe = d.n_experts > 0;
  const bool has_ffn = d.ffn > 0 || moe;
  const float scale = 1.0f / sqrtf((float)hd);
  const int kvf = d.kv_format;
  const bool kv8 = kvf == KD_KV_FP8_E4M3;                // caches hold E4M3 codes
  const size_t kv_rs = (size_t)kv_row_bytes(kvf, hd);   // bytes per cached position of one head
  const int ldqkv = (2 * H + 2 * G) * hd;  // room for the gate rows of gated layers

  RowCaches rc = {};
  for (int b = 0; b < B; ++b) rc.pos[b] = pos[b];
  launch_rope_table(rc, B, hd, d.rope_base, s.cs, st);

  // Residual stream = base (+ add, pending); the pending add is fused into the next norm.
  // A layer whose FFN ends in a resnorm epilogue leaves the next layer's attention input
  // already quantised (codes of x * attn_norm in act, block sums of squares in ss):
  // prenormed, and the QKV product applies 1/rms.
  const float* base = x_in;
  const float* add = nullptr;
  bool prenormed = false;
  const auto norm_fusable = [&](int il) {
    const kd_layer_desc& Ly = m->layers[il];
    return !moe && has_ffn && !Ly.w_up.qs && D <= kNormFuseMax;
  };
  for (int il = 0; il < L; ++il) {
    const kd_layer_desc& Ly = m->layers[il];
    for (int b = 0; b < B; ++b) {
      rc.k[b] = k_base[(size_t)il * B + b];
      rc.v[b] = v_base[(size_t)il * B + b];
    }
    // attn_norm (+ pending residual add) + quantise
    float* res = const_cast<float*>(base);
    if (prenormed) {
      // done by the previous layer's down product
    } else if (add) {
      res = (base == s.xa) ? s.xb : s.xa;
      launch_norm_quant(base, add, Ly.attn_norm, B, D, d.rms_eps, res, nullptr, s.act_qs, s.act_d, st);
    } else {
      launch_norm_quant(base, nullptr, Ly.attn_norm, B, D, d.rms_eps, nullptr, nullptr, s.act_qs, s.act_d, st);
    }
    // res now holds the residual rows entering the layer (written by the previous layer's
    // epilogue or by the norm launch above)
    if (tr && tr->resid && !trace_copy(tr->resid + (size_t)il * B * D, res, sizeof(float) * B * D, st))
      return KD_ERR_HIP;
    if (tr && !trace_codes(tr->q_attn_in, il, s.act_qs, B, D, st)) return KD_ERR_HIP;
    const int att_w = std::max(H * hd, m->ssm_vd);  // the trace's mixer-output record width
    if (Ly.mixer == 1) {
      // gated delta-rule mixer: input projection, conv ring + prep, state step (each row reads
      // ring/state pos % 2 and writes the other), gated norm + quantiser for the out product
      const int nk = d.ssm_n_k, nv = d.ssm_n_v;
      launch_mmvq(Ly.wqkv, s.act_qs, s.act_d, B, s.qkv, m->ssm_nin, st);
      const float* ring_in[KD_MAX_B];
      float* ring_out[KD_MAX_B];
      const float* st_in[KD_MAX_B];
      float* st_out[KD_MAX_B];
      for (int b = 0; b < B; ++b) {
        float* blk = static_cast<float*>(k_base[(size_t)il * B + b]);
        const int par = pos[b] & 1;
        ring_in[b] = blk + par * m->ring_floats;
        ring_out[b] = blk + (1 - par) * m->ring_floats;
        st_in[b] = blk + 2 * m->ring_floats + par * m->state_floats;
        st_out[b] = blk + 2 * m->ring_floats + (1 - par) * m->state_floats;
      }
      launch_ssm_conv_prep(s.qkv, m->ssm_nin, Ly.ssm_conv, d.ssm_d_conv, ring_in, ring_out, Ly.ssm_dt, Ly.ssm_a, B,
                           nk, nv, d.rms_eps, s.lq, s.lk, s.lv, s.lg, s.lb, st);
      launch_gdn_step(s.lq, s.lk, s.lv, s.lg, s.lb, B, nv, st_in, st_out, 1.0f / sqrtf((float)d.ssm_d_state), s.lo,
                      st);
      launch_gated_norm_quant(s.lo, s.qkv + m->ssm_c, m->ssm_nin, Ly.ssm_norm, B, nv, d.rms_eps, s.act_qs, s.act_d,
                              st);
      if (tr && !trace_codes(tr->q_attn_out, il, s.act_qs, B, m->ssm_vd, st, att_w)) return KD_ERR_HIP;
    } else {
    if (Ly.wqkv_pair_rows) {  // the product rotates q/k and appends k/v itself
      launch_mmvq_rope(Ly.wqkv, s.act_qs, s.act_d, B, s.qkv, ldqkv, H, G, hd, s.cs, d.rope_base, rc, capacity, st,
                       prenormed ? s.ss : nullptr, D, d.rms_eps, kv8);
    } else {
      launch_mmvq(Ly.wqkv, s.act_qs, s.act_d, B, s.qkv, ldqkv, st);
      launch_rope_append(s.qkv, ldqkv, B, H, G, hd, s.cs, rc, capacity, true, st, d.rope_base, Ly.q_norm, Ly.k_norm,
                         d.rms_eps, kvf);
    }
    // gated layers: the gate rows follow v in the projection's output row (same stride)
    const float* gate = Ly.attn_gate ? s.qkv + (size_t)(H + 2 * G) * hd : nullptr;
    if (Ly.swa_window > 0) {
      // sliding window: rows holding more than W keys attend the last W through a view of
      // their cache (the row's own key count decides its split, as for full attention)
      int32_t tw[KD_MAX_B];
      RowCaches rw = rc;
      for (int b = 0; b < B; ++b) {
        const int len = pos[b] + 1, off = len > Ly.swa_window ? len - Ly.swa_window : 0;
        tw[b] = len - off;
        rw.k[b] = static_cast<char*>(rc.k[b]) + (size_t)off * kv_rs;
        rw.v[b] = static_cast<char*>(rc.v[b]) + (size_t)off * kv_rs;
      }
      FaPlan pw;
      fa_make_plan(pw, B, H, G, hd, tw, 0);
      launch_fa(pw, s.qkv, ldqkv, rw, capacity, scale, s.attn, s.act_qs, s.act_d, s.fa_ws, st, gate, kvf);
    } else {
      launch_fa(plan, s.qkv, ldqkv, rc, capacity, scale, s.attn, s.act_qs, s.act_d, s.fa_ws, st, gate, kvf);
    }
    if (tr && !trace_codes(tr->q_attn_out, il, s.act_qs, B, H * hd, st, att_w)) return KD_ERR_HIP;
    }  // attention
    if (norm_fusable(il)) {
      // O product + residual add + the FFN RMSNorm's quantiser and sums of squares; the
      // gate/up product applies 1/rms, SwiGLU and the quantiser for down
      float* x1 = (res == s.xa) ? s.xb : s.xa;
      launch_mmvq_resnorm(Ly.wo, s.act_qs, s.act_d, B, res, D, Ly.ffn_norm, x1, s.actn_qs, s.actn_d, s.ss, st);
      if (tr && !trace_codes(tr->q_ffn_in, il, s.actn_qs, B, D, st)) return KD_ERR_HIP;
      launch_mmvq_swiglu(Ly.w_gate, s.actn_qs, s.actn_d, B, s.act2_qs, s.act2_d, st, s.ss, D, d.rms_eps);
      if (tr && !trace_codes(tr->q_ffn_mid, il, s.act2_qs, B, d.ffn, st)) return KD_ERR_HIP;
      if (il + 1 < L && norm_fusable(il + 1) && m->layers[il + 1].wqkv_pair_rows) {
        // down product + residual add + the next layer's attention RMSNorm (its QKV input
        // goes to act, free once the O product has run)
        float* x2 = (x1 == s.xa) ? s.xb : s.xa;
        launch_mmvq_resnorm(Ly.w_down, s.act2_qs, s.act2_d, B, x1, D, m->layers[il + 1].attn_norm, x2, s.act_qs,
                            s.act_d, s.ss, st);
        base = x2;
        add = nullptr;
        prenormed = true;
      } else {
        launch_mmvq(Ly.w_down, s.act2_qs, s.act2_d, B, s.f, D, st);
        base = x1;
        add = s.f;
        prenormed = false;
      }
      continue;
    }
    prenormed = false;
    launch_mmvq(Ly.wo, s.act_qs, s.act_d, B, s.o, D, st);
    if (!has_ffn) {
      base = res;
      add = s.o;
      continue;
    }
    float* x1 = (res == s.xa) ? s.xb : s.xa;
    launch_norm_quant(res, s.o, Ly.ffn_norm, B, D, d.rms_eps, x1, moe ? s.z : nullptr, s.act_qs, s.act_d, st);
    if (tr && !trace_codes(tr->q_ffn_in, il, s.act_qs, B, D, st)) return KD_ERR_HIP;
    if (!moe) {
      const int F = d.ffn;
      if (Ly.w_up.qs) {
        launch_mmvq(Ly.w_gate, s.act_qs, s.act_d, B, s.gu, 2 * F, st);
        launch_mmvq(Ly.w_up, s.act_qs, s.act_d, B, s.gu + F, 2 * F, st);
        launch_swiglu_quant(s.gu, s.gu + F, B, F, 2 * F, nullptr, s.act2_qs, s.act2_d, st);
      } else {  // interleaved gate/up: one product, SwiGLU and quantiser in its epilogue
        launch_mmvq_swiglu(Ly.w_gate, s.act_qs, s.act_d, B, s.act2_qs, s.act2_d, st);
      }
      if (tr && !trace_codes(tr->q_ffn_mid, il, s.act2_qs, B, F, st)) return KD_ERR_HIP;
      launch_mmvq(Ly.w_down, s.act2_qs, s.act2_d, B, s.f, D, st);
    } else {
      const int E = d.n_experts, K = d.n_expert_used, Fe = d.expert_ffn, Fs = d.shared_ffn;
      launch_router(s.z, Ly.router, B, D, E, K, s.ids, s.p, s.rlog, s.count, s.rows, s.pairs, st);
      if (tr && tr->moe_ids && !trace_copy(tr->moe_ids + (size_t)il * B * K, s.ids, sizeof(int32_t) * B * K, st))
        return KD_ERR_HIP;
      if (tr && tr->moe_p && !trace_copy(tr->moe_p + (size_t)il * B * K, s.p, sizeof(float) * B * K, st))
        return KD_ERR_HIP;
      kd_weight eg = Ly.e_gate, eu = Ly.e_up, ed = Ly.e_down;
      ed.n_out = D;
      RowMap dn_map{s.count, s.pairs, s.pairs, E, (long long)n_rowgroups(D) * n_quads(Fe), B * K};
      if (!Ly.e_up.qs) {
        // interleaved experts: one grouped product per layer applies SwiGLU and quantises the
        // (row, rank) rows for the down product; the shared expert likewise
        eg.n_out = 2 * Fe;
        RowMap gu_map{s.count, s.rows, s.pairs, E, (long long)n_rowgroups(2 * Fe) * n_quads(D), B};
        // the shared expert's gate/up rides in the same launch when its matrix is whole groups
        if (mmvq_swiglu_merges(eg, Ly.s_gate)) {
          launch_mmvq_swiglu(eg, s.act_qs, s.act_d, B, s.hq_qs, s.hq_d, st, nullptr, 0, 0.0f, &gu_map, &Ly.s_gate,
                             s.shq_qs, s.shq_d);
        } else {
          launch_mmvq_swiglu(eg, s.act_qs, s.act_d, 0, s.hq_qs, s.hq_d, st, nullptr, 0, 0.0f, &gu_map);
          launch_mmvq_swiglu(Ly.s_gate, s.act_qs, s.act_d, B, s.shq_qs, s.shq_d, st);
        }
        if (tr && !trace_codes(tr->q_ffn_mid, il, s.hq_qs, B * K, Fe, st)) return KD_ERR_HIP;
        if (tr && !trace_codes(tr->q_shared_mid, il, s.shq_qs, B, Fs, st)) return KD_ERR_HIP;
        launch_mmvq(ed, s.hq_qs, s.hq_d, 0, s.yp, D, st, &dn_map);
        // the shared expert's down product writes the layer's output f (experts' rows added)
        launch_mmvq(Ly.s_down, s.shq_qs, s.shq_d, B, s.f, D, st, nullptr, nullptr, s.yp, s.p, K);
      } else {
        RowMap gu_map{s.count, s.rows, s.pairs, E, (long long)n_rowgroups(Fe) * n_quads(D), B};
        eg.n_out = Fe;
        eu.n_out = Fe;
        launch_mmvq(eg, s.act_qs, s.act_d, 0, s.gup, 2 * Fe, st, &gu_map);
        launch_mmvq(eu, s.act_qs, s.act_d, 0, s.gup + Fe, 2 * Fe, st, &gu_map);
        // shared expert gate/up (reads the same Q(z) before it is overwritten)
        launch_mmvq(Ly.s_gate, s.act_qs, s.act_d, B, s.sgu, 2 * Fs, st);
        launch_mmvq(Ly.s_up, s.act_qs, s.act_d, B, s.sgu + Fs, 2 * Fs, st);
        launch_swiglu_quant(s.gup, s.gup + Fe, B * K, Fe, 2 * Fe, nullptr, s.hq_qs, s.hq_d, st);
        if (tr && !trace_codes(tr->q_ffn_mid, il, s.hq_qs, B * K, Fe, st)) return KD_ERR_HIP;
        launch_mmvq(ed, s.hq_qs, s.hq_d, 0, s.yp, D, st, &dn_map);
        launch_swiglu_quant(s.sgu, s.sgu + Fs, B, Fs, 2 * Fs, nullptr, s.act_qs, s.act_d, st);
        if (tr && !trace_codes(tr->q_shared_mid, il, s.act_qs, B, Fs, st)) return KD_ERR_HIP;
        launch_mmvq(Ly.s_down, s.act_qs, s.act_d, B, s.f, D, st, nullptr, nullptr, s.yp, s.p, K);
      }
    }
    base = x1;
    add = s.f;
  }
  if (tr && tr->resid) {  // the residual rows after the last layer
    float* last = tr->resid + (size_t)L * B * D;
    if (add)
      launch_add(base, add, last, (size_t)B * D, st);
    else if (!trace_copy(last, base, sizeof(float) * B * D, st))
      return KD_ERR_HIP;
  }
  // output: [residual add +] final norm [+ quantise + lm_head]
  if (d.vocab > 0) {
    launch_norm_quant(base, add, d.final_norm, B, D, d.rms_eps, nullptr, nullptr, s.act_qs, s.act_d, st);
    if (tr && !trace_codes(tr->q_head_in, 0, s.act_qs, B, D, st)) return KD_ERR_HIP;
    launch_mmvq(d.lm_head, s.act_qs, s.act_d, B, out, d.vocab, st);
  } else if (d.final_norm) {
    launch_norm_quant(base, add, d.final_norm, B, D, d.rms_eps, nullptr, out, nullptr, nullptr, st);
  } else if (add) {
    launch_add(base, add, out, (size_t)B * D, st);
  } else {
    if (hipMemcpyAsync(out, base, sizeof(float) * B * D, hipMemcpyDeviceToDevice, st) != hipSuccess) {
      set_error("kd_decode_step: copy failed");
      return KD_ERR_HIP;
    }
  }
  return check_launch("kd_decode_step");
}

extern "C" kd_status kd_decode_step(const kd_model* m, int32_t B, const float* x_in, const int32_t* pos,
                                    void* const* k_base, void* const* v_base, int32_t capacity, float* out, void* ws,
                                    size_t ws_bytes, void* stream) {
  return decode_step_impl(m, B, x_in, pos, k_base, v_base, capacity, out, ws, ws_bytes, nullptr, stream);
}

extern "C" kd_status kd_debug_decode_step_trace(const kd_model* m, int32_t B, const float* x_in, const int32_t* pos,
                                                void* const* k_base, void* const* v_base, int32_t capacity,
                                                float* out, void* ws, size_t ws_bytes, const kd_step_trace* trace,
                                                void* stream) {
  KD_REQUIRE(trace, KD_ERR_INVALID, "kd_debug_decode_step_trace: null trace");
  return decode_step_impl(m, B, x_in, pos, k_base, v_base, capacity, out, ws, ws_bytes, trace, stream);
}
