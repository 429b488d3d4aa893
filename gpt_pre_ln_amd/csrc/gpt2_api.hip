// C ABI of the GPT-2 Pre-LN forward library (declarations and contract in
// include/gpt2.h).  Host side only: argument checks, the device layouts of
// parameters / workspace / KV cache, and the launch sequence of one forward or
// decode step.  Every step of the computation runs in the kernels of
// rowops.hip, gemm.hip and attention.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/gpt2.h"
#include "attention.h"
#include "backward.h"
#include "gemm.h"
#include "rowops.h"

using namespace gpt2;

namespace {

thread_local std::string g_last_error;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }
inline int round_up_int(int v, int a) { return (v + a - 1) / a * a; }

gpt2_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return GPT2_ERR_HIP;
}

#define GPT2_HIP(call, what)                   \
  do {                                         \
    hipError_t e_ = (call);                    \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// ------------------------------------------------------------------ config

gpt2_status check_config(const gpt2_config* c) {
  if (!c) return GPT2_ERR_INVALID_ARG;
  if (c->vocab_size < 1 || c->n_positions < 1 || c->d_model < 1 || c->n_head < 1 || c->n_layer < 1 ||
      c->d_ff < 1)
    return GPT2_ERR_SHAPE;
  if (c->dtype != GPT2_F32 && c->dtype != GPT2_BF16) return GPT2_ERR_UNSUPPORTED;
  if (c->logits_dtype != GPT2_F32 && c->logits_dtype != GPT2_BF16) return GPT2_ERR_UNSUPPORTED;
  if ((c->activation | c->scale_attn_by_inverse_layer_idx | c->post_ln | c->separate_head) & ~1)
    return GPT2_ERR_UNSUPPORTED;
  if (!(c->ln_eps >= 0.f) || !std::isfinite(c->ln_eps)) return GPT2_ERR_INVALID_ARG;
  if (c->d_model % c->n_head != 0) return GPT2_ERR_SHAPE;
  const int hs = c->d_model / c->n_head;
  if (!(hs == 64 || (hs == 16 && c->dtype == GPT2_F32))) return GPT2_ERR_UNSUPPORTED;
  if (c->d_model % 64 != 0 || c->d_ff % 64 != 0) return GPT2_ERR_UNSUPPORTED;
  if (c->d_model > 2048) return GPT2_ERR_UNSUPPORTED;
  if (c->n_positions > 4096) return GPT2_ERR_UNSUPPORTED;
  if (c->vocab_size > (1 << 24)) return GPT2_ERR_UNSUPPORTED;
  return GPT2_OK;
}

inline size_t esize(const gpt2_config& c) { return c.dtype == GPT2_BF16 ? 2 : 4; }
inline int vocab_pad(const gpt2_config& c) { return round_up_int(c.vocab_size, 256); }
inline int kv_stride(int max_T) { return round_up_int(max_T, 64); }

struct LayerOff {
  size_t ln1_g, ln1_b, w_qkv, b_qkv, w_o, b_o, ln2_g, ln2_b, w_fc, b_fc, w_pr, b_pr;
};

struct ParamLayout {
  size_t wte = 0, wpe = 0, lnf_g = 0, lnf_b = 0, total = 0;
  size_t head = 0;  // [V_pad][D]: wte itself, or the separate head
  std::vector<LayerOff> layers;
};

ParamLayout param_layout(const gpt2_config& c) {
  ParamLayout L;
  const size_t es = esize(c), D = c.d_model, F = c.d_ff;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.wte = take((size_t)vocab_pad(c) * D * es);
  L.wpe = take((size_t)c.n_positions * D * es);
  for (int l = 0; l < c.n_layer; ++l) {
    LayerOff o;
    o.ln1_g = take(D * 4);
    o.ln1_b = take(D * 4);
    o.w_qkv = take(3 * D * D * es);
    o.b_qkv = take(3 * D * 4);
    o.w_o = take(D * D * es);
    o.b_o = take(D * 4);
    o.ln2_g = take(D * 4);
    o.ln2_b = take(D * 4);
    o.w_fc = take(F * D * es);
    o.b_fc = take(F * 4);
    o.w_pr = take(D * F * es);
    o.b_pr = take(D * 4);
    L.layers.push_back(o);
  }
  L.lnf_g = take(D * 4);
  L.lnf_b = take(D * 4);
  L.head = c.separate_head ? take((size_t)vocab_pad(c) * D * es) : L.wte;
  L.total = off;
  return L;
}

size_t blob_floats(const gpt2_config& c) {
  const size_t V = c.vocab_size, P = c.n_positions, D = c.d_model, F = c.d_ff;
  const size_t per_layer = 2 * D + (3 * D * D + 3 * D) + (D * D + D) + 2 * D + (D * F + F) + (F * D + D);
  return V * D + P * D + per_layer * c.n_layer + 2 * D + (c.separate_head ? V * D : 0);
}

// Every tensor of the blob, in blob order, with the place and form of its
// converted copy in the device region (the layout run_init writes).
std::vector<gpt2_param_info> param_table(const gpt2_config& c) {
  const ParamLayout L = param_layout(c);
  const int32_t dt = c.dtype;
  const int64_t V = c.vocab_size, P = c.n_positions, D = c.d_model, F = c.d_ff, Vp = vocab_pad(c);
  std::vector<gpt2_param_info> t;
  int64_t src = 0;
  auto emb = [&](size_t off, int64_t rows, int64_t rows_pad) {  // [rows][D] kept as is, zero rows appended
    t.push_back(gpt2_param_info{src, (int32_t)rows, (int32_t)D, dt, 0, (int64_t)off, D, rows_pad});
    src += rows * D;
  };
  auto mat = [&](size_t off, int64_t K, int64_t N) {  // blob [K][N] -> device [N][K]
    t.push_back(gpt2_param_info{src, (int32_t)K, (int32_t)N, dt, 1, (int64_t)off, K, N});
    src += K * N;
  };
  auto vec = [&](size_t off, int64_t n) {
    t.push_back(gpt2_param_info{src, 1, (int32_t)n, GPT2_F32, 0, (int64_t)off, n, 1});
    src += n;
  };
  emb(L.wte, V, Vp);
  emb(L.wpe, P, P);
  for (const LayerOff& o : L.layers) {
    vec(o.ln1_g, D);
    vec(o.ln1_b, D);
    mat(o.w_qkv, D, 3 * D);
    vec(o.b_qkv, 3 * D);
    mat(o.w_o, D, D);
    vec(o.b_o, D);
    vec(o.ln2_g, D);
    vec(o.ln2_b, D);
    mat(o.w_fc, D, F);
    vec(o.b_fc, F);
    mat(o.w_pr, F, D);
    vec(o.b_pr, D);
  }
  vec(L.lnf_g, D);
  vec(L.lnf_b, D);
  if (c.separate_head) emb(L.head, V, Vp);
  return t;
}

// Tile shape per GEMM: 256x256 only where there are enough tiles to fill the
// 256 CUs many times over (the lm_head); then 128x192 (8 waves, one block
// per CU) or 128x96 (2 blocks per CU) where their grids fill whole rounds;
// 128x128 (2 blocks per CU) or 64x128 (3 blocks per CU) otherwise.
GemmTile pick_tile(int M, int N, int K) {
  if (M <= 32) return kTile32x64;
  if (M <= 64) return kTile64x64;
  const long tiles256 = (long)((M + 255) / 256) * ((N + 255) / 256);
  if (tiles256 >= 8 * 256) return kTile256x256;
  // 128x192 with 8 waves of 64x48 (one block per CU, 80 KB of LDS) where
  // its grid fills at least three whole rounds of the 256 CUs: per CU it
  // streams 320 operand rows per k step for the same 8 wave tiles that two
  // 128x96 blocks feed with 448.  GPT-2 small at B*T = 8192: qkv (768 tiles)
  // and c_fc (1,024); standalone 38.4 -> 33.6 us and 47.0 -> 45.0 us.  The
  // one-round c_proj grids measured slower on it (17.9 -> 18.8 and 42.6 ->
  // 44.5 us) and stay below.
  {
    const long t192 = (long)((M + 127) / 128) * ((N + 191) / 192);
    if (N % 192 == 0 && t192 % 256 == 0 && t192 >= 3 * 256) return kTile128x192;
  }
  // 128x96 (2 blocks per CU) where its grid fills whole rounds of the 512
  // block slots and the 128x128 grid does not: per CU round it streams 448
  // operand rows against 512 for 128x128 and 576 for 64x128.  GPT-2 small at
  // B*T = 8192: attn.c_proj and mlp.c_proj (512 tiles, 1 round; qkv's 1,536
  // tiles too, before the 128x192 rule); measured 5-7 % faster per launch
  // than 64x128 or 128x128 on those shapes.
  {
    constexpr long kSlots = 2 * 256;
    const long t96 = (long)((M + 127) / 128) * ((N + 95) / 96);
    const long t128 = (long)((M + 127) / 128) * ((N + 127) / 128);
    if (N % 96 == 0 && t96 % kSlots == 0 && t128 % kSlots != 0) return kTile128x96;
  }
  // Short k loops (K <= 1024): 64x128 tiles run 3 blocks per CU against 2 for
  // 128x128; take the one whose busiest CU computes fewer output elements
  // (ties to the larger tile).  GPT-2 small: qkv and attn.c_proj take 64x128
  // (the 128x128 grids leave the last round a quarter or half full); with
  // K = 3072 the smaller tile's extra operand traffic outweighs the balance
  // (mlp.c_proj measured 6 % slower), so long k loops keep 128x128.
  if (K <= 1024) {
    constexpr long kCUs = 256;
    const long t128 = (long)((M + 127) / 128) * ((N + 127) / 128);
    const long t64 = (long)((M + 63) / 64) * ((N + 127) / 128);
    const long w128 = (t128 + kCUs - 1) / kCUs * 128 * 128, w64 = (t64 + kCUs - 1) / kCUs * 64 * 128;
    if (w64 < w128) return kTile64x128;
  }
  return kTile128x128;
}

struct WsLayout {
  size_t x, h, q, k, vt, a, u, part, rpart;
  // next-token loss (lm_head partials, label logits, per-position losses):
  // placed over q .. rpart, which are dead once ln_f has run
  size_t ce_part, ce_tgt, ce_loss;
  int ce_nseg;
  // generation loop: the token chosen at one step, read by the next
  size_t gen_tok;
  size_t total;
};

// decode_only: the layout of a decode step alone, without the prefill key and
// value buffers (a decode step reads and appends to the caller's cache).
WsLayout ws_layout(const gpt2_config& c, int B, int T, bool decode_only = false) {
  WsLayout W;
  const size_t es = esize(c), D = c.d_model, F = c.d_ff, M = (size_t)B * T;
  const size_t Tp = kv_stride(T);
  const int hs = c.d_model / c.n_head;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  W.x = take(M * D * 4);
  W.h = take(M * D * es);
  W.q = take(M * D * es);
  W.k = take(decode_only ? 0 : (size_t)B * Tp * D * es);
  W.vt = take(decode_only ? 0 : (size_t)B * Tp * D * es);
  W.a = take(M * D * es);
  W.u = take(M * F * es);
  W.part = take(decode_partials_floats(B, c.n_head, hs) * 4);
  // split-K partials of the decode step's residual projections (at most 32 rows)
  const int ks = std::max(skinny_splits(c.d_model, (int)es), skinny_splits(c.d_ff, (int)es));
  W.rpart = take((size_t)ks * std::min<size_t>(M, 32) * D * 4);
  W.gen_tok = take(M * 4);
  const size_t end = off;
  off = W.q;
  W.ce_nseg = vocab_pad(c) / gemm_slice_width(pick_tile((int)M, vocab_pad(c), c.d_model));
  W.ce_part = take(M * W.ce_nseg * sizeof(float2));
  W.ce_tgt = take(M * 4);
  W.ce_loss = take(M * 4);
  W.total = std::max(end, off);
  return W;
}

size_t kv_layer_bytes(const gpt2_config& c, int B, int max_T) {
  return 2 * (size_t)B * kv_stride(max_T) * c.d_model * esize(c);
}

// ------------------------------------------------------------------ allocation-free decode

// Scratch of gpt2_decode_step_noalloc: the decode step's activations and
// partial results, in a device array that exists for the life of the process
// (one per GPU), for callers that cannot allocate.  Host code never passes the
// array's name to a kernel or a copy: that name is a host-side stand-in, and
// the device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (set up on first use).
gpt2_status scratch_of_current_device(char** out) {
  int dev = -1;
  GPT2_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return GPT2_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    GPT2_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return GPT2_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return GPT2_OK;
}

// ------------------------------------------------------------------ timing

enum KernelClass { kEmbed = 0, kLN = 1, kQKV = 2, kAttn = 3, kOProj = 4, kFC = 5, kMLPProj = 6, kLMHead = 7 };
constexpr int kMaxTimed = 4096;

}  // namespace

struct gpt2_model {
  gpt2_config cfg;
  char* params;
  size_t param_bytes;
  char* ws;
  size_t ws_bytes;
  ParamLayout lay;
  float* trace = nullptr;
  size_t trace_floats = 0;
  int32_t* id_flag = nullptr;  // set to 1 by the embedding when an id was outside [0, V)
  bool timing_on = false;
  int timing_class = -1;
  std::vector<hipEvent_t> ev;  // 2 per launch
  int n_timed = 0;
  bool timing_overflow = false;
};

namespace {

struct TimedScope {
  gpt2_model* m;
  hipStream_t s;
  bool active;
  TimedScope(gpt2_model* m_, int cls, hipStream_t s_) : m(m_), s(s_), active(false) {
    if (m->timing_on && m->timing_class == cls) {
      if (m->n_timed < kMaxTimed) {
        active = true;
        // a failed record surfaces as an error of gpt2_timing_read (the
        // elapsed time of an unrecorded event is an error there)
        (void)hipEventRecord(m->ev[2 * m->n_timed], s);
      } else {
        m->timing_overflow = true;
      }
    }
  }
  ~TimedScope() {
    if (active) {
      (void)hipEventRecord(m->ev[2 * m->n_timed + 1], s);
      ++m->n_timed;
    }
  }
};

template <typename T>
const T* pp(const gpt2_model* m, size_t off) {
  return reinterpret_cast<const T*>(m->params + off);
}
const float* pf(const gpt2_model* m, size_t off) { return reinterpret_cast<const float*>(m->params + off); }

inline int ilog2(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Block projections: the one-kernel skinny path for at most 32 rows, the tiled
// MFMA kernel otherwise.
template <typename T, class Epi>
hipError_t proj_gemm(const T* A, const T* Bw, int M, int N, int K, const Epi& epi, hipStream_t st) {
  if (M <= 32) return launch_gemm_skinny<T>(A, Bw, M, N, K, K, K, epi, st);
  return launch_gemm<T>(pick_tile(M, N, K), A, Bw, M, N, K, K, K, epi, st);
}

// c_fc with its GELU epilogue, the form (0: gelu_new, 1: erf) chosen here
// once so that each kernel carries one form only.
template <typename T>
hipError_t c_fc_gemm(int erf, const T* h, const T* w_fc, const float* b_fc, T* u, int M, int F, int D,
                     hipStream_t st) {
  if (erf) return proj_gemm<T>(h, w_fc, M, F, D, EpiGelu<T, true>{b_fc, u, F}, st);
  return proj_gemm<T>(h, w_fc, M, F, D, EpiGelu<T, false>{b_fc, u, F}, st);
}

// Weight read-ahead.  Inside a forward a layer's weight matrices have dropped
// out of the caches by the time they are used again (the activations stream
// several hundred MB between two uses), and a GEMM that meets its weights cold
// reads them from all eight XCDs at once: the qkv GEMM of GPT-2 small at B=8
// T=1024 takes 59 us cold against 47 us after one plain read of its weights.
// The LayerNorm before each pair of GEMMs therefore also reads their weights
// (it is bound by HBM and a few MB more cost it ~2 us).  Measured
// alternatives: a separate read kernel before each GEMM (0.08 ms slower per
// forward) and reads on a second stream overlapping the preceding kernel
// (slower still: they contend with it).
// lm_head: logits = h @ wte^T (tied, no bias), stored as cfg.logits_dtype in
// rows of ld elements.  With ld >= vocab_pad the rows are written in whole,
// the padding columns receiving the zero logits of the zero padding rows of
// the embedding: no per-column test at the vocabulary edge, and rows that
// start on 128-byte boundaries when ld is a multiple of 64 (the lm_head of
// GPT-2 small at B=8 T=1024: 738 -> 722 us for whole rows, from 769 us with
// unaligned rows of vocab_size elements; standalone, bf16 logits).
template <typename T>
hipError_t launch_lm_head(gpt2_model* m, const T* h, void* logits, int64_t ld, int M, hipStream_t st) {
  const gpt2_config& c = m->cfg;
  const int D = c.d_model, Vp = vocab_pad(c);
  const int n_store = ld >= Vp ? Vp : c.vocab_size;
  const GemmTile tile = pick_tile(M, Vp, D);
  if (c.logits_dtype == GPT2_BF16) {
    EpiLogits<bf16_t> e{static_cast<bf16_t*>(logits), (int)ld, n_store};
    return launch_gemm<T>(tile, h, pp<T>(m, m->lay.head), M, Vp, D, D, D, e, st);
  }
  EpiLogits<float> e{static_cast<float*>(logits), (int)ld, n_store};
  return launch_gemm<T>(tile, h, pp<T>(m, m->lay.head), M, Vp, D, D, D, e, st);
}

// ------------------------------------------------------------------ forward

// Outputs of the next-token loss (gpt2_forward_loss).
struct LossOut {
  const int32_t* labels;  // [B][T]
  float* token_loss;      // [B][T-1] or null
  float* mean;            // [1] or null
};

template <typename T>
gpt2_status run_forward(gpt2_model* m, const int32_t* tokens, int B, int T_seq, void* logits, int64_t logits_ld,
                        float* hidden, gpt2_kv_view* kv, const LossOut* loss, hipStream_t st) {
  const gpt2_config& c = m->cfg;
  const int D = c.d_model, H = c.n_head, hs = D / H, F = c.d_ff, V = c.vocab_size;
  const int M = B * T_seq;
  const WsLayout W = ws_layout(c, B, T_seq);
  float* x = reinterpret_cast<float*>(m->ws + W.x);
  T* h = reinterpret_cast<T*>(m->ws + W.h);
  T* q = reinterpret_cast<T*>(m->ws + W.q);
  T* a = reinterpret_cast<T*>(m->ws + W.a);
  T* u = reinterpret_cast<T*>(m->ws + W.u);
  const int kvT = kv ? kv_stride(kv->max_T) : kv_stride(T_seq);
  const float q_scale = 1.0f / std::sqrt((float)hs);
  // Weight read-ahead for the tiled GEMMs (the skinny ones read each weight once
  // anyway): ln_1 reads c_attn.w .. attn.c_proj.w, ln_2 mlp.c_fc.w .. mlp.c_proj.w
  // (adjacent in the parameter region), in bytes rounded down to 16.
  const bool pre = M > 32;
  auto span = [&](size_t first, size_t last, size_t last_elems) {
    return ((last + last_elems * sizeof(T)) - first) / 16 * 16;
  };

  // Post-LN: the first block's attention reads the embeddings themselves (an
  // operand copy of x); later blocks read the output of the previous ln_2.
  const bool post = c.post_ln != 0;
  if (post) {
    TimedScope ts(m, kEmbed, st);
    GPT2_HIP(launch_embed<T>(tokens, pp<T>(m, m->lay.wte), pp<T>(m, m->lay.wpe), x, M, T_seq, 0, D, V, m->id_flag, st), "embed");
  } else {
    // Pre-LN: the embedding and the first block's ln_1 in one pass
    const LayerOff& o0 = m->lay.layers[0];
    TimedScope ts(m, kEmbed, st);
    GPT2_HIP(launch_embed_layernorm<T>(tokens, pp<T>(m, m->lay.wte), pp<T>(m, m->lay.wpe), x, M, T_seq, 0, D, V,
                                       m->id_flag, pf(m, o0.ln1_g), pf(m, o0.ln1_b), h, c.ln_eps, st,
                                       pre ? m->params + o0.w_qkv : nullptr, span(o0.w_qkv, o0.w_o, (size_t)D * D)),
             "embed + ln_1");
  }
  if (post) GPT2_HIP(launch_convert<T>(x, h, (size_t)M * D, (size_t)M * D, st), "post-ln input");
  for (int l = 0; l < c.n_layer; ++l) {
    const LayerOff& o = m->lay.layers[l];
    T* kl;
    T* vtl;
    if (kv) {
      char* base = reinterpret_cast<char*>(kv->d_kv) + (size_t)l * kv_layer_bytes(c, kv->B, kv->max_T);
      kl = reinterpret_cast<T*>(base);
      vtl = reinterpret_cast<T*>(base + kv_layer_bytes(c, kv->B, kv->max_T) / 2);
    } else {
      kl = reinterpret_cast<T*>(m->ws + W.k);
      vtl = reinterpret_cast<T*>(m->ws + W.vt);
    }
    const float q_scale_l = c.scale_attn_by_inverse_layer_idx ? q_scale / (float)(l + 1) : q_scale;
    if (!post && l > 0) {  // layer 0's ln_1 ran with the embedding
      TimedScope ts(m, kLN, st);
      GPT2_HIP(launch_layernorm<T>(x, pf(m, o.ln1_g), pf(m, o.ln1_b), h, nullptr, M, D, c.ln_eps, st,
                                   pre ? m->params + o.w_qkv : nullptr, span(o.w_qkv, o.w_o, (size_t)D * D)),
               "ln_1");
    }
    {
      TimedScope ts(m, kQKV, st);
      EpiQKV<T> e{pf(m, o.b_qkv), q, kl, vtl, FastDiv(T_seq), FastDiv(D), 0, kvT, H, ilog2(hs), q_scale_l, M};
      GPT2_HIP(proj_gemm<T>(h, pp<T>(m, o.w_qkv), M, 3 * D, D, e, st), "c_attn");
    }
    {
      TimedScope ts(m, kAttn, st);
      GPT2_HIP(launch_attention_prefill<T>(q, kl, vtl, a, B, H, T_seq, kvT, hs, st), "attention");
    }
    {
      TimedScope ts(m, kOProj, st);
      EpiResidual e{pf(m, o.b_o), x, D};
      GPT2_HIP(proj_gemm<T>(a, pp<T>(m, o.w_o), M, D, D, e, st), "attn.c_proj");
    }
    {
      // Pre-LN: h = ln_2(x).  Post-LN: x = ln_1(x) in place, h its operand copy.
      TimedScope ts(m, kLN, st);
      GPT2_HIP(launch_layernorm<T>(x, pf(m, post ? o.ln1_g : o.ln2_g), pf(m, post ? o.ln1_b : o.ln2_b), h,
                                   post ? x : nullptr, M, D, c.ln_eps, st, pre ? m->params + o.w_fc : nullptr,
                                   span(o.w_fc, o.w_pr, (size_t)D * F)),
               post ? "ln_1" : "ln_2");
    }
    {
      TimedScope ts(m, kFC, st);
      GPT2_HIP(c_fc_gemm<T>(c.activation, h, pp<T>(m, o.w_fc), pf(m, o.b_fc), u, M, F, D, st), "c_fc");
    }
    {
      TimedScope ts(m, kMLPProj, st);
      EpiResidual e{pf(m, o.b_pr), x, D};
      GPT2_HIP(proj_gemm<T>(u, pp<T>(m, o.w_pr), M, D, F, e, st), "mlp.c_proj");
    }
    if (post) {
      // x = ln_2(x) in place, h the next block's attention input
      const bool next = l + 1 < c.n_layer;
      const LayerOff& on = m->lay.layers[next ? l + 1 : l];
      TimedScope ts(m, kLN, st);
      GPT2_HIP(launch_layernorm<T>(x, pf(m, o.ln2_g), pf(m, o.ln2_b), h, x, M, D, c.ln_eps, st,
                                   pre && next ? m->params + on.w_qkv : nullptr,
                                   span(on.w_qkv, on.w_o, (size_t)D * D)),
               "ln_2");
    }
    if (m->trace && (size_t)(l + 1) * M * D <= m->trace_floats) {
      GPT2_HIP(hipMemcpyAsync(m->trace + (size_t)l * M * D, x, (size_t)M * D * 4, hipMemcpyDeviceToDevice, st),
               "trace copy");
    }
  }
  {
    TimedScope ts(m, kLN, st);
    GPT2_HIP(launch_layernorm<T>(x, pf(m, m->lay.lnf_g), pf(m, m->lay.lnf_b), h, hidden, M, D, c.ln_eps, st), "ln_f");
  }
  if (logits) {
    TimedScope ts(m, kLMHead, st);
    GPT2_HIP(launch_lm_head<T>(m, h, logits, logits_ld, M, st), "lm_head");
  }
  if (loss) {
    // lm_head with the cross-entropy epilogue: per-slice (max, sum exp) and
    // the label logits, then one wave per position and one block for the mean
    float2* part = reinterpret_cast<float2*>(m->ws + W.ce_part);
    float* tgt = reinterpret_cast<float*>(m->ws + W.ce_tgt);
    float* per = loss->token_loss ? loss->token_loss : reinterpret_cast<float*>(m->ws + W.ce_loss);
    {
      TimedScope ts(m, kLMHead, st);
      const GemmTile tile = pick_tile(M, vocab_pad(c), D);
      EpiCE e{part, W.ce_nseg, loss->labels, FastDiv((uint32_t)T_seq), V, tgt};
      GPT2_HIP(launch_gemm<T>(tile, h, pp<T>(m, m->lay.head), M, vocab_pad(c), D, D, D, e, st), "lm_head loss");
    }
    GPT2_HIP(launch_ce_rows(part, W.ce_nseg, tgt, loss->labels, B, T_seq, V, per, st), "loss rows");
    if (loss->mean) GPT2_HIP(launch_ce_mean(per, loss->labels, B, T_seq, loss->mean, st), "loss mean");
  }
  if (kv) kv->past_len = T_seq;
  return GPT2_OK;
}

// Output of a generation step (gpt2_generate): the greedy token of row b goes
// to out[b * stride + col] and to next[b].
struct GenOut {
  int32_t* out;
  int stride, col;
  int32_t* next;
  bool sample = false;  // draw from softmax(logits / temperature) instead of the arg-max
  uint64_t seed_mix = 0;  // splitmix64(seed)
  float inv_temp = 1.f;
};

// ws (optional): run on this scratch region, laid out by
// ws_layout(.., decode_only = true), instead of the handle's workspace.
template <typename T>
gpt2_status run_decode(gpt2_model* m, gpt2_kv_view* kv, const int32_t* tokens, void* logits, const GenOut* gen,
                       hipStream_t st, char* ws = nullptr) {
  const gpt2_config& c = m->cfg;
  const int D = c.d_model, H = c.n_head, hs = D / H, F = c.d_ff, V = c.vocab_size;
  const int B = kv->B, M = B, pos = kv->past_len;
  const WsLayout W = ws_layout(c, B, 1, ws != nullptr);
  char* const wsb = ws ? ws : m->ws;
  float* x = reinterpret_cast<float*>(wsb + W.x);
  T* h = reinterpret_cast<T*>(wsb + W.h);
  T* q = reinterpret_cast<T*>(wsb + W.q);
  T* a = reinterpret_cast<T*>(wsb + W.a);
  T* u = reinterpret_cast<T*>(wsb + W.u);
  float* part = reinterpret_cast<float*>(wsb + W.part);
  // Up to 32 rows the residual projections (attn.c_proj, mlp.c_proj) write
  // split-K partial products and the LayerNorm that follows each adds them,
  // the bias and the residual stream, writes x back and normalises: no reduce
  // launch.  More rows take the tiled GEMM with the residual epilogue.
  const bool split = M <= 32;
  float* rpart = reinterpret_cast<float*>(wsb + W.rpart);
  const int ks_o = skinny_splits(D, sizeof(T)), ks_p = skinny_splits(F, sizeof(T));
  const float* pending_bias = nullptr;  // mlp.c_proj bias of the previous layer, when partials are pending
  const int kvT = kv_stride(kv->max_T);
  const float q_scale = 1.0f / std::sqrt((float)hs);

  // Post-LN: each LayerNorm follows a residual add (ln_1 after attn.c_proj,
  // ln_2 after mlp.c_proj) and also writes the normalised row back to x; the
  // first block's attention reads an operand copy of the embeddings.
  const bool post = c.post_ln != 0;
  if (post)
    GPT2_HIP(launch_embed<T>(tokens, pp<T>(m, m->lay.wte), pp<T>(m, m->lay.wpe), x, M, 1, pos, D, V, m->id_flag, st),
             "embed");
  else  // Pre-LN: the embedding and the first block's ln_1 in one pass
    GPT2_HIP(launch_embed_layernorm<T>(tokens, pp<T>(m, m->lay.wte), pp<T>(m, m->lay.wpe), x, M, 1, pos, D, V,
                                       m->id_flag, pf(m, m->lay.layers[0].ln1_g), pf(m, m->lay.layers[0].ln1_b), h,
                                       c.ln_eps, st, nullptr, 0),
             "embed + ln_1");
  if (post) GPT2_HIP(launch_convert<T>(x, h, (size_t)M * D, (size_t)M * D, st), "post-ln input");
  for (int l = 0; l < c.n_layer; ++l) {
    const LayerOff& o = m->lay.layers[l];
    char* base = reinterpret_cast<char*>(kv->d_kv) + (size_t)l * kv_layer_bytes(c, B, kv->max_T);
    T* kl = reinterpret_cast<T*>(base);
    T* vtl = reinterpret_cast<T*>(base + kv_layer_bytes(c, B, kv->max_T) / 2);
    const float q_scale_l = c.scale_attn_by_inverse_layer_idx ? q_scale / (float)(l + 1) : q_scale;
    if (!post && l > 0)  // layer 0's ln_1 ran with the embedding
      GPT2_HIP(launch_layernorm<T>(x, pf(m, o.ln1_g), pf(m, o.ln1_b), h, nullptr, M, D, c.ln_eps, st, nullptr, 0,
                                   pending_bias ? rpart : nullptr, ks_p, pending_bias),
               "ln_1");
    {
      EpiQKV<T> e{pf(m, o.b_qkv), q, kl, vtl, FastDiv(1), FastDiv(D), pos, kvT, H, ilog2(hs), q_scale_l, M};
      GPT2_HIP(proj_gemm<T>(h, pp<T>(m, o.w_qkv), M, 3 * D, D, e, st), "c_attn");
    }
    GPT2_HIP(launch_attention_decode<T>(q, kl, vtl, a, part, B, H, pos + 1, kvT, hs, st), "attention decode");
    if (split) {
      GPT2_HIP(launch_gemm_skinny_splitk<T>(a, pp<T>(m, o.w_o), M, D, D, D, D, rpart, st), "attn.c_proj");
    } else {
      EpiResidual e{pf(m, o.b_o), x, D};
      GPT2_HIP(proj_gemm<T>(a, pp<T>(m, o.w_o), M, D, D, e, st), "attn.c_proj");
    }
    // Pre-LN: h = ln_2(x + partials).  Post-LN: x = ln_1(x + partials), h its copy.
    GPT2_HIP(launch_layernorm<T>(x, pf(m, post ? o.ln1_g : o.ln2_g), pf(m, post ? o.ln1_b : o.ln2_b), h,
                                 post ? x : nullptr, M, D, c.ln_eps, st, nullptr, 0, split ? rpart : nullptr, ks_o,
                                 pf(m, o.b_o)),
             post ? "ln_1" : "ln_2");
    {
      GPT2_HIP(c_fc_gemm<T>(c.activation, h, pp<T>(m, o.w_fc), pf(m, o.b_fc), u, M, F, D, st), "c_fc");
    }
    if (split) {
      GPT2_HIP(launch_gemm_skinny_splitk<T>(u, pp<T>(m, o.w_pr), M, D, F, F, F, rpart, st), "mlp.c_proj");
      pending_bias = pf(m, o.b_pr);
    } else {
      EpiResidual e{pf(m, o.b_pr), x, D};
      GPT2_HIP(proj_gemm<T>(u, pp<T>(m, o.w_pr), M, D, F, e, st), "mlp.c_proj");
    }
    if (post) {
      // x = ln_2(x + partials) in place; h is the next block's attention input
      GPT2_HIP(launch_layernorm<T>(x, pf(m, o.ln2_g), pf(m, o.ln2_b), h, x, M, D, c.ln_eps, st, nullptr, 0,
                                   pending_bias ? rpart : nullptr, ks_p, pending_bias),
               "ln_2");
      pending_bias = nullptr;
    }
  }
  GPT2_HIP(launch_layernorm<T>(x, pf(m, m->lay.lnf_g), pf(m, m->lay.lnf_b), h, nullptr, M, D, c.ln_eps, st, nullptr, 0,
                               pending_bias ? rpart : nullptr, ks_p, pending_bias),
           "ln_f");
  if (gen) {
    // lm_head with the arg-max epilogue (no logits stored), then one wave per row
    int2* apart = reinterpret_cast<int2*>(wsb + W.ce_part);
    if (gen->sample) {
      EpiSample e{apart, W.ce_nseg, V, gen->seed_mix, pos, gen->inv_temp};
      GPT2_HIP(launch_gemm<T>(pick_tile(M, vocab_pad(c), D), h, pp<T>(m, m->lay.head), M, vocab_pad(c), D, D, D, e,
                              st),
               "lm_head sample");
    } else {
      EpiArgmax e{apart, W.ce_nseg, V};
      GPT2_HIP(launch_gemm<T>(pick_tile(M, vocab_pad(c), D), h, pp<T>(m, m->lay.head), M, vocab_pad(c), D, D, D, e,
                              st),
               "lm_head argmax");
    }
    GPT2_HIP(launch_argmax_rows(apart, W.ce_nseg, M, V, gen->out + gen->col, gen->stride, gen->next, st), "argmax");
  } else {
    GPT2_HIP(launch_lm_head<T>(m, h, logits, c.vocab_size, M, st), "lm_head");
  }
  kv->past_len = pos + 1;
  return GPT2_OK;
}

// ------------------------------------------------------------------ block backward

// Backward workspace (caller-owned, gpt2_block_backward_workspace_bytes):
// the recomputed forward of the block and the gradient temporaries.
struct BwdLayout {
  size_t h1, q, k, vt, lse, dvec, a, xh, h2, g, u, dyt, wt_qkv, wt_o, wt_fc, wt_pr, dg, dh, dxh, dxht, da, dqkv,
      dqkvt, ta, tb, mu, rstd, part, wpart, total;
};

// Weight-gradient products [Mr][N] contract over the Mp = B*T (padded)
// positions: few output tiles, a long k loop.  Split K into the smallest
// power of two of slices that gives at least 512 blocks (at most 16 slices,
// each at least 512 deep and a multiple of 64).
int wgrad_splits(int Mr, int N, int Mp) {
  int bm = 128, bn = 128;
  switch (pick_tile(Mr, N, Mp)) {
    case kTile256x256: bm = bn = 256; break;
    case kTile64x64: bm = bn = 64; break;
    case kTile32x64: bm = 32, bn = 64; break;
    case kTile64x128: bm = 64, bn = 128; break;
    case kTile128x96: bm = 128, bn = 96; break;
    case kTile128x192: bm = 128, bn = 192; break;
    default: break;
  }
  const long tiles = (long)((Mr + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int n64 = Mp / 64;
  int s = 1;
  while (s < 16 && tiles * s < 512 && n64 % (2 * s) == 0 && Mp / (2 * s) >= 512) s *= 2;
  return s;
}

BwdLayout bwd_layout(const gpt2_config& c, int B, int T) {
  BwdLayout L;
  const size_t es = esize(c), D = c.d_model, F = c.d_ff, M = (size_t)B * T, Mp = round_up_int((int)M, 64);
  const size_t Tp = kv_stride(T), BH = (size_t)B * c.n_head, hs = D / c.n_head;
  const size_t wide = std::max(F, 3 * D);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.h1 = take(M * D * es);
  L.q = take(M * D * es);
  L.k = take(BH * Tp * hs * es);
  L.vt = take(BH * Tp * hs * es);
  L.lse = take(BH * T * 4);
  L.dvec = take(BH * T * 4);
  L.a = take(M * D * es);
  L.xh = take(M * D * 4);
  L.h2 = take(M * D * es);
  L.g = take(M * F * 4);
  L.u = take(M * F * es);
  L.dyt = take(M * D * es);
  L.wt_qkv = take(3 * D * D * es);
  L.wt_o = take(D * D * es);
  L.wt_fc = take(D * F * es);
  L.wt_pr = take(F * D * es);
  L.dg = take(M * F * es);
  L.dh = take(M * D * 4);
  L.dxh = take(M * D * 4);
  L.dxht = take(M * D * es);
  L.da = take(M * D * es);
  L.dqkv = take(M * 3 * D * 4);
  L.dqkvt = take(M * 3 * D * es);
  L.ta = take(wide * Mp * es);
  L.tb = take(wide * Mp * es);
  L.mu = take(M * 4);
  L.rstd = take(M * 4);
  // first-pass partials of the eight column sums (biases, gamma, beta), kept
  // until one grouped second pass at the end: D + F + 2D + D + 3D + 2D columns
  L.part = take(colsum_partial_floats((int)(9 * D + F)) * 4);
  size_t wp = 0;
  const int Di = (int)D, Fi = (int)F, Mpi = (int)Mp;
  for (const auto& mn : {std::pair<int, int>{Fi, Di}, {Di, Fi}, {Di, Di}, {Di, 3 * Di}}) {
    const int s = wgrad_splits(mn.first, mn.second, Mpi);
    if (s > 1) wp = std::max(wp, (size_t)s * mn.first * mn.second);
  }
  L.wpart = take(wp * 4);
  L.total = off;
  return L;
}

// Backward of Pre-LN block l (dpshk.com llm.c notes 5.3; the block's forward
// as in russellluo.com "GPT-2 Block" and pwwt.cn GPT2Block / GPT2Attention /
// GPT2MLP), taken in reverse:
//   forward recomputed from x: h1 = LN_1(x), q|k|v, attention (keeping each
//   query's log-sum-exp), x_h = x + a W_o + b_o, h2 = LN_2(x_h),
//   g = h2 W_fc + b_fc (kept in fp32), u = act(g);
//   MLP: dg = (dy W_pr^T) act'(g), dW_pr = u^T dy, dW_fc = h2^T dg,
//        dh2 = dg W_fc^T;  x_h gradient = dy + LN_2 backward(dh2);
//   attention: dW_o = a^T dx_h, da = dx_h W_o^T, attention backward -> dq|dk|dv,
//        dW_qkv = h1^T dqkv, dh1 = dqkv W_qkv^T;  dx = dx_h + LN_1 backward(dh1).
// Products run on the GEMM kernel (C = A B^T, both operands contiguous in
// the contraction): weight-side operands from transposed copies of this
// layer's weights; the weight gradients read the activations as stored
// (K-major operands, bf16 with B*T a multiple of 64) or else transposed
// copies padded to a multiple of 64 rows.  Bias, gamma and beta gradients
// are column sums.
template <typename T>
gpt2_status run_block_backward(gpt2_model* m, int l, int B, int T_seq, const float* x, const float* dy, float* dx,
                               float* grads, char* ws, hipStream_t st) {
  const gpt2_config& c = m->cfg;
  const int D = c.d_model, H = c.n_head, hs = D / H, F = c.d_ff;
  const int M = B * T_seq, Mp = round_up_int(M, 64), Tp = kv_stride(T_seq);
  const BwdLayout L = bwd_layout(c, B, T_seq);
  const LayerOff& o = m->lay.layers[l];
  auto wp = [&](size_t off) { return reinterpret_cast<T*>(ws + off); };
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  T *h1 = wp(L.h1), *q = wp(L.q), *kk = wp(L.k), *vt = wp(L.vt), *a = wp(L.a), *h2 = wp(L.h2), *u = wp(L.u);
  T *dyt = wp(L.dyt), *dg = wp(L.dg), *dxht = wp(L.dxht), *da = wp(L.da), *dqkvt = wp(L.dqkvt);
  T *ta = wp(L.ta), *tb = wp(L.tb);
  T *wt_qkv = wp(L.wt_qkv), *wt_o = wp(L.wt_o), *wt_fc = wp(L.wt_fc), *wt_pr = wp(L.wt_pr);
  float *lse = fp(L.lse), *dvec = fp(L.dvec), *xh = fp(L.xh), *gpre = fp(L.g), *dh = fp(L.dh), *dxh = fp(L.dxh);
  float *dqkv = fp(L.dqkv), *mu = fp(L.mu), *rstd = fp(L.rstd), *part = fp(L.part);
  float q_scale = 1.0f / std::sqrt((float)hs);
  if (c.scale_attn_by_inverse_layer_idx) q_scale /= (float)(l + 1);
  // gradient slices of this layer, in the blob's order
  const size_t G_ln1w = 0, G_ln1b = D, G_qkvw = 2 * (size_t)D, G_qkvb = G_qkvw + 3 * (size_t)D * D,
               G_ow = G_qkvb + 3 * D, G_ob = G_ow + (size_t)D * D, G_ln2w = G_ob + D, G_ln2b = G_ln2w + D,
               G_fcw = G_ln2b + D, G_fcb = G_fcw + (size_t)D * F, G_prw = G_fcb + F, G_prb = G_prw + (size_t)F * D;
  auto gemm_f32 = [&](const T* A, const T* Bm, int Mr, int N, int K, float* out, int ldo) {
    return launch_gemm<T>(pick_tile(Mr, N, K), A, Bm, Mr, N, K, K, K, EpiStore<float>{out, ldo}, st);
  };
  // weight gradient [Mr][N] = A[Mr][Mp] B[N][Mp]^T, split over K when it has few tiles
  float* wpart = fp(L.wpart);
  auto wgrad = [&](const T* A, const T* Bm, int Mr, int N, float* out) -> hipError_t {
    const int s = wgrad_splits(Mr, N, Mp);
    if (s == 1) return gemm_f32(A, Bm, Mr, N, Mp, out, N);
    hipError_t e = launch_gemm_splitk<T>(pick_tile(Mr, N, Mp), A, Bm, Mr, N, Mp / s, Mp, Mp, s,
                                         EpiStore<float>{wpart, N, (size_t)Mr * N}, st);
    if (e != hipSuccess) return e;
    return launch_sum_splits(wpart, s, (size_t)Mr * N, out, st);
  };
  // bf16 with whole 64-position k steps: the weight gradient reads both
  // activations as stored ([M][Mr] and [M][N], K-major) through transposing
  // LDS reads, so no transposed copies (the product itself runs ~30 % slower
  // than on K-contiguous copies: 47 -> 62 us for the GPT-2 small shapes, the
  // k-loop being bound by its LDS reads, against ~10 us per 8192 x 768
  // transpose and ~23 us per 8192 x 3072 one saved); otherwise transpose
  // into the padded [Mr][Mp] / [N][Mp] copies and take the plain product.
  auto wgrad_act = [&](const T* Xa, int Mr, const T* Xb, int N, float* out) -> hipError_t {
    if constexpr (std::is_same_v<T, bf16_t>) {
      if (M % 64 == 0 && Mr % 8 == 0 && N % 8 == 0 && pick_tile(Mr, N, Mp) == kTile128x128) {
        const int s = wgrad_splits(Mr, N, Mp);
        if (s == 1) return launch_gemm_kmajor(Xa, Xb, Mr, N, M, Mr, N, 1, EpiStore<float>{out, N}, st);
        hipError_t e = launch_gemm_kmajor(Xa, Xb, Mr, N, M / s, Mr, N, s, EpiStore<float>{wpart, N, (size_t)Mr * N},
                                          st);
        if (e != hipSuccess) return e;
        return launch_sum_splits(wpart, s, (size_t)Mr * N, out, st);
      }
    }
    hipError_t e = launch_transpose<T, T>(Xa, M, Mr, ta, Mp, st);
    if (e != hipSuccess) return e;
    e = launch_transpose<T, T>(Xb, M, N, tb, Mp, st);
    if (e != hipSuccess) return e;
    return wgrad(ta, tb, Mr, N, out);
  };

  // transposed copies of this layer's weights ([out][in] -> [in][out])
  GPT2_HIP((launch_transpose<T, T>(pp<T>(m, o.w_qkv), 3 * D, D, wt_qkv, 3 * D, st)), "bwd transpose w_qkv");
  GPT2_HIP((launch_transpose<T, T>(pp<T>(m, o.w_o), D, D, wt_o, D, st)), "bwd transpose w_o");
  GPT2_HIP((launch_transpose<T, T>(pp<T>(m, o.w_fc), F, D, wt_fc, F, st)), "bwd transpose w_fc");
  GPT2_HIP((launch_transpose<T, T>(pp<T>(m, o.w_pr), D, F, wt_pr, D, st)), "bwd transpose w_pr");

  // forward of the block, keeping what the backward reads
  GPT2_HIP(launch_layernorm<T>(const_cast<float*>(x), pf(m, o.ln1_g), pf(m, o.ln1_b), h1, nullptr, M, D, c.ln_eps, st),
           "bwd ln_1");
  {
    EpiQKV<T> e{pf(m, o.b_qkv), q, kk, vt, FastDiv(T_seq), FastDiv(D), 0, Tp, H, ilog2(hs), q_scale, M};
    GPT2_HIP(launch_gemm<T>(pick_tile(M, 3 * D, D), h1, pp<T>(m, o.w_qkv), M, 3 * D, D, D, D, e, st), "bwd c_attn");
  }
  GPT2_HIP(launch_attention_prefill<T>(q, kk, vt, a, B, H, T_seq, Tp, hs, st, lse), "bwd attention");
  {
    EpiResidual e{pf(m, o.b_o), xh, D, x};  // xh = x + attn.c_proj(a)
    GPT2_HIP(launch_gemm<T>(pick_tile(M, D, D), a, pp<T>(m, o.w_o), M, D, D, D, D, e, st), "bwd attn.c_proj");
  }
  GPT2_HIP(launch_layernorm<T>(xh, pf(m, o.ln2_g), pf(m, o.ln2_b), h2, nullptr, M, D, c.ln_eps, st), "bwd ln_2");
  {
    auto fc = [&](auto erf) {
      EpiGeluSave<T, decltype(erf)::value> e{pf(m, o.b_fc), u, gpre, F};
      return launch_gemm<T>(pick_tile(M, F, D), h2, pp<T>(m, o.w_fc), M, F, D, D, D, e, st);
    };
    GPT2_HIP(c.activation ? fc(std::true_type{}) : fc(std::false_type{}), "bwd c_fc");
  }

  // MLP
  GPT2_HIP(launch_convert<T>(dy, dyt, (size_t)M * D, (size_t)M * D, st), "bwd dy");
  {
    auto du = [&](auto erf) {
      EpiGeluBwd<T, decltype(erf)::value> e{gpre, dg, F};
      return launch_gemm<T>(pick_tile(M, F, D), dyt, wt_pr, M, F, D, D, D, e, st);
    };
    GPT2_HIP(c.activation ? du(std::true_type{}) : du(std::false_type{}), "bwd du");
  }
  // column sums: first passes into their own partial slots now (their sources
  // are overwritten later), one grouped second pass at the end
  ColsumJob cjobs[kMaxColsumJobs];
  int n_cjobs = 0;
  float* pslot = part;
  auto colsum_slot = [&](int N, float* out) {
    float* p = pslot;
    pslot += colsum_partial_floats(N);
    cjobs[n_cjobs++] = ColsumJob{p, out, N};
    return p;
  };
  GPT2_HIP(launch_colsum_partial<float>(dy, M, D, colsum_slot(D, grads + G_prb), st), "bwd db_pr");
  GPT2_HIP(wgrad_act(u, F, dyt, D, grads + G_prw), "bwd dW_pr");
  GPT2_HIP(launch_colsum_partial<T>(dg, M, F, colsum_slot(F, grads + G_fcb), st), "bwd db_fc");
  GPT2_HIP(wgrad_act(h2, D, dg, F, grads + G_fcw), "bwd dW_fc");
  GPT2_HIP(gemm_f32(dg, wt_fc, M, D, F, dh, D), "bwd dh2");
  GPT2_HIP(launch_layernorm_backward<T>(xh, dh, pf(m, o.ln2_g), dy, dxh, dxht, mu, rstd, M, D, c.ln_eps, st),
           "bwd ln_2 backward");
  {
    float* pw = colsum_slot(D, grads + G_ln2w);
    float* pb = colsum_slot(D, grads + G_ln2b);
    GPT2_HIP(launch_colsum_partial<float>(dh, M, D, pw, st, xh, mu, rstd, pb), "bwd dgamma_2, dbeta_2");
  }

  // attention
  GPT2_HIP(launch_colsum_partial<float>(dxh, M, D, colsum_slot(D, grads + G_ob), st), "bwd db_o");
  GPT2_HIP(wgrad_act(a, D, dxht, D, grads + G_ow), "bwd dW_o");
  GPT2_HIP(launch_gemm<T>(pick_tile(M, D, D), dxht, wt_o, M, D, D, D, D, EpiStore<T>{da, D}, st), "bwd da");
  GPT2_HIP(launch_attention_backward<T>(q, kk, vt, a, da, lse, dvec, dqkv, B, H, T_seq, Tp, hs, q_scale, st),
           "bwd attention backward");
  GPT2_HIP(launch_colsum_partial<float>(dqkv, M, 3 * D, colsum_slot(3 * D, grads + G_qkvb), st), "bwd db_qkv");
  GPT2_HIP(launch_convert<T>(dqkv, dqkvt, (size_t)M * 3 * D, (size_t)M * 3 * D, st), "bwd dqkv");
  GPT2_HIP(wgrad_act(h1, D, dqkvt, 3 * D, grads + G_qkvw), "bwd dW_qkv");
  GPT2_HIP(gemm_f32(dqkvt, wt_qkv, M, D, 3 * D, dh, D), "bwd dh1");
  GPT2_HIP(launch_layernorm_backward<T>(x, dh, pf(m, o.ln1_g), dxh, dx, static_cast<T*>(nullptr), mu, rstd, M, D,
                                        c.ln_eps, st),
           "bwd ln_1 backward");
  {
    float* pw = colsum_slot(D, grads + G_ln1w);
    float* pb = colsum_slot(D, grads + G_ln1b);
    GPT2_HIP(launch_colsum_partial<float>(dh, M, D, pw, st, x, mu, rstd, pb), "bwd dgamma_1, dbeta_1");
  }
  GPT2_HIP(launch_colsum_final(cjobs, n_cjobs, st), "bwd column sums");
  return GPT2_OK;
}

template <typename T>
gpt2_status run_init(gpt2_model* m, const float* blob, hipStream_t st) {
  const gpt2_config& c = m->cfg;
  const size_t V = c.vocab_size, P = c.n_positions, D = c.d_model, F = c.d_ff;
  size_t src = 0;  // float offset into the blob
  auto mat = [&](size_t dst_off, size_t K, size_t N) -> gpt2_status {  // blob [K][N] -> device [N][K]
    GPT2_HIP(launch_transpose_convert<T>(blob + src, reinterpret_cast<T*>(m->params + dst_off), (int)K, (int)N,
                                         (int)N, st),
             "init transpose");
    src += K * N;
    return GPT2_OK;
  };
  auto vec = [&](size_t dst_off, size_t n) -> gpt2_status {
    GPT2_HIP(hipMemcpyAsync(m->params + dst_off, blob + src, n * 4, hipMemcpyDeviceToDevice, st), "init copy");
    src += n;
    return GPT2_OK;
  };
  gpt2_status s;
  GPT2_HIP(launch_convert<T>(blob + src, reinterpret_cast<T*>(m->params + m->lay.wte), V * D,
                             (size_t)vocab_pad(c) * D, st),
           "init wte");
  src += V * D;
  GPT2_HIP(launch_convert<T>(blob + src, reinterpret_cast<T*>(m->params + m->lay.wpe), P * D, P * D, st),
           "init wpe");
  src += P * D;
  for (int l = 0; l < c.n_layer; ++l) {
    const LayerOff& o = m->lay.layers[l];
    if ((s = vec(o.ln1_g, D)) || (s = vec(o.ln1_b, D)) || (s = mat(o.w_qkv, D, 3 * D)) || (s = vec(o.b_qkv, 3 * D)) ||
        (s = mat(o.w_o, D, D)) || (s = vec(o.b_o, D)) || (s = vec(o.ln2_g, D)) || (s = vec(o.ln2_b, D)) ||
        (s = mat(o.w_fc, D, F)) || (s = vec(o.b_fc, F)) || (s = mat(o.w_pr, F, D)) || (s = vec(o.b_pr, D)))
      return s;
  }
  if ((s = vec(m->lay.lnf_g, D)) || (s = vec(m->lay.lnf_b, D))) return s;
  if (c.separate_head) {
    GPT2_HIP(launch_convert<T>(blob + src, reinterpret_cast<T*>(m->params + m->lay.head), V * D,
                               (size_t)vocab_pad(c) * D, st),
             "init lm_head");
    src += V * D;
  }
  return GPT2_OK;
}

}  // namespace

// ======================================================================= C ABI

extern "C" {

const char* gpt2_status_string(gpt2_status s) {
  switch (s) {
    case GPT2_OK: return "ok";
    case GPT2_ERR_INVALID_ARG: return "invalid argument";
    case GPT2_ERR_SHAPE: return "shape out of range";
    case GPT2_ERR_CAPACITY: return "kv cache capacity exceeded";
    case GPT2_ERR_WORKSPACE: return "workspace or parameter region too small";
    case GPT2_ERR_UNSUPPORTED: return "unsupported configuration";
    case GPT2_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* gpt2_last_error(void) { return g_last_error.c_str(); }

#ifndef GPT2_SOURCE_HASH
#define GPT2_SOURCE_HASH "unknown"
#endif
const char* gpt2_source_hash(void) { return GPT2_SOURCE_HASH; }

gpt2_status gpt2_param_blob_floats(const gpt2_config* cfg, size_t* n) {
  gpt2_status s = check_config(cfg);
  if (s) return s;
  if (!n) return GPT2_ERR_INVALID_ARG;
  *n = blob_floats(*cfg);
  return GPT2_OK;
}

gpt2_status gpt2_param_bytes(const gpt2_config* cfg, size_t* bytes) {
  gpt2_status s = check_config(cfg);
  if (s) return s;
  if (!bytes) return GPT2_ERR_INVALID_ARG;
  *bytes = param_layout(*cfg).total;
  return GPT2_OK;
}

gpt2_status gpt2_param_tensor_count(const gpt2_config* cfg, int32_t* n) {
  gpt2_status s = check_config(cfg);
  if (s) return s;
  if (!n) return GPT2_ERR_INVALID_ARG;
  *n = (int32_t)param_table(*cfg).size();
  return GPT2_OK;
}

gpt2_status gpt2_param_tensor(const gpt2_config* cfg, int32_t index, gpt2_param_info* info) {
  gpt2_status s = check_config(cfg);
  if (s) return s;
  if (!info) return GPT2_ERR_INVALID_ARG;
  const std::vector<gpt2_param_info> t = param_table(*cfg);
  if (index < 0 || (size_t)index >= t.size()) return GPT2_ERR_SHAPE;
  *info = t[index];
  return GPT2_OK;
}

gpt2_status gpt2_kv_stride(const gpt2_config* cfg, int32_t max_T, int32_t* stride) {
  gpt2_status s = check_config(cfg);
  if (s) return s;
  if (!stride) return GPT2_ERR_INVALID_ARG;
  if (max_T < 1 || max_T > cfg->n_positions) return GPT2_ERR_SHAPE;
  *stride = kv_stride(max_T);
  return GPT2_OK;
}

gpt2_status gpt2_workspace_bytes(const gpt2_config* cfg, int32_t B, int32_t T, size_t* bytes) {
  gpt2_status s = check_config(cfg);
  if (s) return s;
  if (!bytes) return GPT2_ERR_INVALID_ARG;
  if (B < 1 || T < 1 || T > cfg->n_positions || (int64_t)B * T > (1 << 24)) return GPT2_ERR_SHAPE;
  *bytes = ws_layout(*cfg, B, T).total;
  return GPT2_OK;
}

gpt2_status gpt2_kv_cache_bytes(const gpt2_config* cfg, int32_t B, int32_t max_T, size_t* bytes) {
  gpt2_status s = check_config(cfg);
  if (s) return s;
  if (!bytes) return GPT2_ERR_INVALID_ARG;
  if (B < 1 || max_T < 1 || max_T > cfg->n_positions) return GPT2_ERR_SHAPE;
  *bytes = (size_t)cfg->n_layer * kv_layer_bytes(*cfg, B, max_T);
  return GPT2_OK;
}

gpt2_status gpt2_create(const gpt2_config* cfg, void* d_params, size_t param_bytes, void* d_workspace,
                        size_t ws_bytes, gpt2_model** out) {
  gpt2_status s = check_config(cfg);
  if (s) return s;
  if (!out || !d_params || !d_workspace) return GPT2_ERR_INVALID_ARG;
  if (!aligned(d_params, kAlign) || !aligned(d_workspace, kAlign)) return GPT2_ERR_INVALID_ARG;
  ParamLayout lay = param_layout(*cfg);
  if (param_bytes < lay.total) return GPT2_ERR_WORKSPACE;
  if (ws_bytes < ws_layout(*cfg, 1, 1).total) return GPT2_ERR_WORKSPACE;
  gpt2_model* m = new gpt2_model();
  m->cfg = *cfg;
  m->params = static_cast<char*>(d_params);
  m->param_bytes = param_bytes;
  m->ws = static_cast<char*>(d_workspace);
  m->ws_bytes = ws_bytes;
  m->lay = std::move(lay);
  *out = m;
  return GPT2_OK;
}

void gpt2_destroy(gpt2_model* m) {
  if (!m) return;
  for (hipEvent_t e : m->ev) (void)hipEventDestroy(e);  // nothing to do about a failure here
  delete m;
}

gpt2_status gpt2_init_params(gpt2_model* m, const float* d_blob, size_t n, void* stream) {
  if (!m || !d_blob) return GPT2_ERR_INVALID_ARG;
  if (!aligned(d_blob, 4)) return GPT2_ERR_INVALID_ARG;
  if (n != blob_floats(m->cfg)) return GPT2_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return m->cfg.dtype == GPT2_BF16 ? run_init<bf16_t>(m, d_blob, st) : run_init<float>(m, d_blob, st);
}

gpt2_status gpt2_forward(gpt2_model* m, const int32_t* tokens, int32_t B, int32_t T, void* logits, float* hidden,
                         gpt2_kv_view* kv, void* stream) {
  if (!m) return GPT2_ERR_INVALID_ARG;
  return gpt2_forward_strided(m, tokens, B, T, logits, m->cfg.vocab_size, hidden, kv, stream);
}

gpt2_status gpt2_logits_padded_ld(const gpt2_config* cfg, int64_t* ld) {
  if (!cfg || !ld) return GPT2_ERR_INVALID_ARG;
  if (cfg->vocab_size < 1) return GPT2_ERR_SHAPE;
  *ld = vocab_pad(*cfg);
  return GPT2_OK;
}

gpt2_status gpt2_forward_strided(gpt2_model* m, const int32_t* tokens, int32_t B, int32_t T, void* logits,
                                 int64_t logits_ld, float* hidden, gpt2_kv_view* kv, void* stream) {
  if (!m || !tokens) return GPT2_ERR_INVALID_ARG;
  if (logits && (logits_ld < m->cfg.vocab_size || logits_ld > INT32_MAX)) return GPT2_ERR_SHAPE;
  if (B < 1 || T < 1 || T > m->cfg.n_positions || (int64_t)B * T > (1 << 24)) return GPT2_ERR_SHAPE;
  const size_t lsz = m->cfg.logits_dtype == GPT2_BF16 ? 2 : 4;
  if (!aligned(tokens, 4) || (logits && !aligned(logits, lsz)) || (hidden && !aligned(hidden, 16)))
    return GPT2_ERR_INVALID_ARG;
  if (ws_layout(m->cfg, B, T).total > m->ws_bytes) return GPT2_ERR_WORKSPACE;
  if (kv) {
    if (!kv->d_kv || !aligned(kv->d_kv, kAlign)) return GPT2_ERR_INVALID_ARG;
    if (kv->B != B) return GPT2_ERR_SHAPE;
    if (kv->max_T < T || kv->max_T > m->cfg.n_positions) return GPT2_ERR_CAPACITY;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  return m->cfg.dtype == GPT2_BF16 ? run_forward<bf16_t>(m, tokens, B, T, logits, logits_ld, hidden, kv, nullptr, st)
                                   : run_forward<float>(m, tokens, B, T, logits, logits_ld, hidden, kv, nullptr, st);
}

gpt2_status gpt2_forward_loss(gpt2_model* m, const int32_t* tokens, const int32_t* labels, int32_t B, int32_t T,
                              float* token_loss, float* mean_loss, void* stream) {
  if (!m || !tokens || (!token_loss && !mean_loss)) return GPT2_ERR_INVALID_ARG;
  if (B < 1 || T < 2 || T > m->cfg.n_positions || (int64_t)B * T > (1 << 24)) return GPT2_ERR_SHAPE;
  if (!aligned(tokens, 4) || (labels && !aligned(labels, 4)) || (token_loss && !aligned(token_loss, 4)) ||
      (mean_loss && !aligned(mean_loss, 4)))
    return GPT2_ERR_INVALID_ARG;
  if (ws_layout(m->cfg, B, T).total > m->ws_bytes) return GPT2_ERR_WORKSPACE;
  const LossOut lo{labels ? labels : tokens, token_loss, mean_loss};
  hipStream_t st = static_cast<hipStream_t>(stream);
  return m->cfg.dtype == GPT2_BF16 ? run_forward<bf16_t>(m, tokens, B, T, nullptr, 0, nullptr, nullptr, &lo, st)
                                   : run_forward<float>(m, tokens, B, T, nullptr, 0, nullptr, nullptr, &lo, st);
}

gpt2_status gpt2_decode_step(gpt2_model* m, gpt2_kv_view* kv, const int32_t* tokens, void* logits, void* stream) {
  if (!m || !kv || !tokens || !logits || !kv->d_kv) return GPT2_ERR_INVALID_ARG;
  const size_t lsz = m->cfg.logits_dtype == GPT2_BF16 ? 2 : 4;
  if (!aligned(kv->d_kv, kAlign) || !aligned(tokens, 4) || !aligned(logits, lsz)) return GPT2_ERR_INVALID_ARG;
  if (kv->B < 1 || kv->max_T < 1 || kv->max_T > m->cfg.n_positions) return GPT2_ERR_SHAPE;
  if (kv->past_len < 0) return GPT2_ERR_SHAPE;
  if (kv->past_len >= kv->max_T) return GPT2_ERR_CAPACITY;
  if (ws_layout(m->cfg, kv->B, 1).total > m->ws_bytes) return GPT2_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return m->cfg.dtype == GPT2_BF16 ? run_decode<bf16_t>(m, kv, tokens, logits, nullptr, st)
                                   : run_decode<float>(m, kv, tokens, logits, nullptr, st);
}

gpt2_status gpt2_decode_step_noalloc(gpt2_model* m, gpt2_kv_view* kv, const int32_t* tokens, void* logits,
                                     void* stream) {
  if (!m || !kv || !tokens || !logits || !kv->d_kv) return GPT2_ERR_INVALID_ARG;
  const size_t lsz = m->cfg.logits_dtype == GPT2_BF16 ? 2 : 4;
  if (!aligned(kv->d_kv, kAlign) || !aligned(tokens, 4) || !aligned(logits, lsz)) return GPT2_ERR_INVALID_ARG;
  if (kv->B < 1 || kv->max_T < 1 || kv->max_T > m->cfg.n_positions) return GPT2_ERR_SHAPE;
  if (kv->past_len < 0) return GPT2_ERR_SHAPE;
  if (kv->past_len >= kv->max_T) return GPT2_ERR_CAPACITY;
  if (ws_layout(m->cfg, kv->B, 1, true).total > kNoAllocScratchBytes) {
    g_last_error = "gpt2_decode_step_noalloc: the step needs " +
                   std::to_string(ws_layout(m->cfg, kv->B, 1, true).total) + " bytes of scratch, more than the " +
                   std::to_string(kNoAllocScratchBytes) + " the library holds per device";
    return GPT2_ERR_WORKSPACE;
  }
  char* ws = nullptr;
  gpt2_status s = scratch_of_current_device(&ws);
  if (s != GPT2_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return m->cfg.dtype == GPT2_BF16 ? run_decode<bf16_t>(m, kv, tokens, logits, nullptr, st, ws)
                                   : run_decode<float>(m, kv, tokens, logits, nullptr, st, ws);
}

gpt2_status gpt2_decode_scratch_bytes(const gpt2_config* cfg, int32_t B, size_t* bytes, size_t* limit) {
  gpt2_status s = check_config(cfg);
  if (s) return s;
  if (!bytes && !limit) return GPT2_ERR_INVALID_ARG;
  if (B < 1 || B > (1 << 24)) return GPT2_ERR_SHAPE;
  if (bytes) *bytes = ws_layout(*cfg, B, 1, true).total;
  if (limit) *limit = kNoAllocScratchBytes;
  return GPT2_OK;
}

gpt2_status gpt2_generate_sample(gpt2_model* m, gpt2_kv_view* kv, const int32_t* tokens, int32_t n_steps,
                                 float temperature, uint64_t seed, int32_t* out, void* stream) {
  if (!(temperature >= 0.f) || !std::isfinite(temperature)) return GPT2_ERR_INVALID_ARG;
  if (temperature == 0.f) return gpt2_generate(m, kv, tokens, n_steps, out, stream);
  if (!m || !kv || !tokens || !out || !kv->d_kv) return GPT2_ERR_INVALID_ARG;
  if (!aligned(kv->d_kv, kAlign) || !aligned(tokens, 4) || !aligned(out, 4)) return GPT2_ERR_INVALID_ARG;
  if (n_steps < 1) return GPT2_ERR_SHAPE;
  if (kv->B < 1 || kv->max_T < 1 || kv->max_T > m->cfg.n_positions) return GPT2_ERR_SHAPE;
  if (kv->past_len < 0) return GPT2_ERR_SHAPE;
  if ((int64_t)kv->past_len + n_steps > kv->max_T) return GPT2_ERR_CAPACITY;
  const WsLayout W = ws_layout(m->cfg, kv->B, 1);
  if (W.total > m->ws_bytes) return GPT2_ERR_WORKSPACE;
  int32_t* next = reinterpret_cast<int32_t*>(m->ws + W.gen_tok);
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int i = 0; i < n_steps; ++i) {
    GenOut g{out, n_steps, i, next};
    g.sample = true;
    g.seed_mix = splitmix64(seed);
    g.inv_temp = 1.0f / temperature;
    const int32_t* in = i == 0 ? tokens : next;
    const gpt2_status s = m->cfg.dtype == GPT2_BF16 ? run_decode<bf16_t>(m, kv, in, nullptr, &g, st)
                                                    : run_decode<float>(m, kv, in, nullptr, &g, st);
    if (s != GPT2_OK) return s;
  }
  return GPT2_OK;
}

gpt2_status gpt2_generate(gpt2_model* m, gpt2_kv_view* kv, const int32_t* tokens, int32_t n_steps, int32_t* out,
                          void* stream) {
  if (!m || !kv || !tokens || !out || !kv->d_kv) return GPT2_ERR_INVALID_ARG;
  if (!aligned(kv->d_kv, kAlign) || !aligned(tokens, 4) || !aligned(out, 4)) return GPT2_ERR_INVALID_ARG;
  if (n_steps < 1) return GPT2_ERR_SHAPE;
  if (kv->B < 1 || kv->max_T < 1 || kv->max_T > m->cfg.n_positions) return GPT2_ERR_SHAPE;
  if (kv->past_len < 0) return GPT2_ERR_SHAPE;
  if ((int64_t)kv->past_len + n_steps > kv->max_T) return GPT2_ERR_CAPACITY;
  const WsLayout W = ws_layout(m->cfg, kv->B, 1);
  if (W.total > m->ws_bytes) return GPT2_ERR_WORKSPACE;
  int32_t* next = reinterpret_cast<int32_t*>(m->ws + W.gen_tok);
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int i = 0; i < n_steps; ++i) {
    const GenOut g{out, n_steps, i, next};
    const int32_t* in = i == 0 ? tokens : next;
    const gpt2_status s = m->cfg.dtype == GPT2_BF16 ? run_decode<bf16_t>(m, kv, in, nullptr, &g, st)
                                                    : run_decode<float>(m, kv, in, nullptr, &g, st);
    if (s != GPT2_OK) return s;
  }
  return GPT2_OK;
}

gpt2_status gpt2_block_backward_workspace_bytes(const gpt2_config* cfg, int32_t B, int32_t T, size_t* bytes) {
  gpt2_status s = check_config(cfg);
  if (s) return s;
  if (!bytes) return GPT2_ERR_INVALID_ARG;
  if (B < 1 || T < 1 || T > cfg->n_positions || (int64_t)B * T > (1 << 24)) return GPT2_ERR_SHAPE;
  *bytes = bwd_layout(*cfg, B, T).total;
  return GPT2_OK;
}

gpt2_status gpt2_block_backward(gpt2_model* m, int32_t layer, int32_t B, int32_t T, const float* x, const float* dy,
                                float* dx, float* grads, void* ws, size_t ws_bytes, void* stream) {
  if (!m || !x || !dy || !dx || !grads || !ws) return GPT2_ERR_INVALID_ARG;
  if (m->cfg.post_ln) return GPT2_ERR_UNSUPPORTED;
  if (layer < 0 || layer >= m->cfg.n_layer) return GPT2_ERR_SHAPE;
  if (B < 1 || T < 1 || T > m->cfg.n_positions || (int64_t)B * T > (1 << 24)) return GPT2_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16) || !aligned(grads, 16) || !aligned(ws, kAlign))
    return GPT2_ERR_INVALID_ARG;
  if (dx == x || dx == dy) return GPT2_ERR_INVALID_ARG;
  if (bwd_layout(m->cfg, B, T).total > ws_bytes) return GPT2_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  return m->cfg.dtype == GPT2_BF16 ? run_block_backward<bf16_t>(m, layer, B, T, x, dy, dx, grads, w, st)
                                   : run_block_backward<float>(m, layer, B, T, x, dy, dx, grads, w, st);
}

gpt2_status gpt2_set_id_check(gpt2_model* m, int32_t* d_flag) {
  if (!m) return GPT2_ERR_INVALID_ARG;
  if (d_flag && !aligned(d_flag, 4)) return GPT2_ERR_INVALID_ARG;
  m->id_flag = d_flag;
  return GPT2_OK;
}

gpt2_status gpt2_set_trace(gpt2_model* m, float* d_trace, size_t n) {
  if (!m) return GPT2_ERR_INVALID_ARG;
  if (d_trace && !aligned(d_trace, 4)) return GPT2_ERR_INVALID_ARG;
  m->trace = d_trace;
  m->trace_floats = d_trace ? n : 0;
  return GPT2_OK;
}

gpt2_status gpt2_timing_enable(gpt2_model* m, int32_t which, int32_t on) {
  if (!m || which < 0 || which > kLMHead) return GPT2_ERR_INVALID_ARG;
  if (on && m->ev.empty()) {
    m->ev.resize(2 * kMaxTimed);
    for (auto& e : m->ev) GPT2_HIP(hipEventCreate(&e), "hipEventCreate");
  }
  m->timing_on = on != 0;
  m->timing_class = which;
  m->n_timed = 0;
  m->timing_overflow = false;
  return GPT2_OK;
}

gpt2_status gpt2_timing_read(gpt2_model* m, double* total_ms, int32_t* launches) {
  if (!m || !total_ms || !launches) return GPT2_ERR_INVALID_ARG;
  double tot = 0.0;
  for (int i = 0; i < m->n_timed; ++i) {
    GPT2_HIP(hipEventSynchronize(m->ev[2 * i + 1]), "hipEventSynchronize");
    float ms = 0.f;
    GPT2_HIP(hipEventElapsedTime(&ms, m->ev[2 * i], m->ev[2 * i + 1]), "hipEventElapsedTime");
    tot += ms;
  }
  *total_ms = tot;
  *launches = m->n_timed;
  m->n_timed = 0;
  m->timing_overflow = false;
  return GPT2_OK;
}

}  // extern "C"
