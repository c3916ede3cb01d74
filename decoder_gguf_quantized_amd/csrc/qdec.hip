// libqdec: runtime and C ABI of the MI355X quantized decoder.
//
// The model struct owns repacked weights, the f32 KV cache and the workspace;
// each ABI call validates its arguments on the host, then enqueues the step's
// kernels on the caller's stream and returns.  Handle / status / poison rules
// follow tessl `python/README.md` ("Handle ownership, closing and errors", "How
// the buffers cross"); the forward pass follows the Qwen3 walkthrough Steps 2-9
// and the qwen3 architecture file on Synsema "Local inference and architectures".
#include "../../include/qdec.h"


#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>
#include <cstdlib>
#include <new>
#include <string>
#include <mutex>
#include <thread>
#include <unordered_map>
#include <vector>

#include "attention.hpp"
#include "common.hpp"
#include "gemm.hpp"
#include "gemv.hpp"
#include "misc.hpp"
#include "dispatch.hpp"

using namespace qd;

namespace {

thread_local std::string g_err;


void set_err(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
}

struct Mat {
  int type = -1;
  int rows = 0, cols = 0, nblk = 0;
  uint8_t* qs = nullptr;   // quants (or f32 values for F32)
  uint16_t* d = nullptr;   // fp16 scales (K-quants: per-sub-block scale words)
  uint32_t* sd = nullptr;  // K-quants: per-super-block scales
  double gguf_bytes = 0;   // bytes of the tensor in GGUF layout (what a step streams)
};

struct Layer {
  float* attn_norm = nullptr;
  float* q_norm = nullptr;
  float* k_norm = nullptr;
  float* post_attn = nullptr;
  float* ffn_norm = nullptr;
  float* post_ffw = nullptr;
  float* qkv_bias = nullptr;  // [nqkv] q|k|v projection bias, or null
  Mat qkv, o, gu, down;
  bool qkv_split = false;  // q, k, v of different types: three matrices instead of qkv
  Mat qkv_part[3];
  bool global = true;
};

struct NameRef {
  const Mat* mat = nullptr;
  int row_off = 0, rows = 0, cols = 0, pair = 0;
  const float* vec = nullptr;
};

struct KRec {
  const char* cls;
  hipEvent_t a, b;
  double bytes, flops;
};

bool is_quant(int t) { return t == kQ8_0 || t == kQ4_0; }  // 32-value blocks with an fp16 scale
bool is_kquant(int t) { return t == kQ4_K || t == kQ6_K; }  // 256-value super-blocks
bool known_type(int t) { return t == kF32 || is_quant(t) || is_kquant(t); }
int64_t blk_bytes(int t) { return t == kQ8_0 ? 34 : 18; }
int64_t super_bytes(int t) { return t == kQ4_K ? 144 : 210; }
int64_t nblocks(int64_t cols) { return (cols + 31) / 32; }
int64_t tensor_bytes(int t, int64_t rows, int64_t cols) {
  if (t == kF32) return rows * cols * 4;
  if (is_kquant(t)) return rows * (cols / 256) * super_bytes(t);
  return rows * nblocks(cols) * blk_bytes(t);
}

void hipck(hipError_t e, const char* what) {
  if (e != hipSuccess) throw HipError{std::string(what) + ": " + hipGetErrorString(e)};
}

}  // namespace

struct qdec_model {
  qdec_config cfg{};
  int max_seqs = 0, max_ctx = 0;
  int qd = 0, kd = 0, nqkv = 0, Fp = 0;
  std::vector<Layer> layers;
  Mat embd, out_w;
  bool tied = true;
  float* output_norm = nullptr;
  float2* rope_g = nullptr;  // [max_ctx][hd/2] (cos, sin), full-attention layers
  float2* rope_l = nullptr;  // same for sliding-window layers
  float2* rope_cur = nullptr;  // [2][max_seqs][hd/2]: rows of rope_g / rope_l at each decode position
  int prefill_prec = QDEC_PREFILL_F32;  // operand precision of the prefill GEMMs
  float* kc = nullptr;
  float* vc = nullptr;
  size_t kv_layer = 0;  // floats of the largest layer of one cache
  std::vector<size_t> kv_off;  // float offset of each layer in kc / vc
  std::vector<int> kv_ring;    // a contiguous window layer's ring: log2 of its positions, 0 = none
  bool ring_on = true;         // window layers keep a ring (qdec_kv_ring)
  int ws_T = 0;
  float *x = nullptr, *h = nullptr, *qkv = nullptr, *q = nullptr, *a = nullptr, *m = nullptr, *y = nullptr;
  float* x2 = nullptr;  // second residual buffer (decode with sandwich norms)
  float* acc = nullptr;   // decode attention's accumulators: two layer parities, each
                          // kAccCopies blocks of [max_seqs][n_head][head_dim] (o) then
                          // [max_seqs][n_head] (l)
  size_t acc_blk = 0;     // floats per block (a parity holds kAccCopies blocks)
  int chunk = 0, nchunk = 0;
  int chunk_base = 0;  // decode chunk for a paged cache: the load-time chunk rounded up to a
                       // power of two (then capped at the page size)
  float* s_v = nullptr;
  int* s_i = nullptr;
  float* am_v = nullptr;  // [am_n] the LM head's per-wave greedy choices (one row)
  int* am_i = nullptr;
  int am_n = 0;           // the most waves an LM-head launch can have (set at load)
  uint32_t* cut_key = nullptr;  // [max_seqs] top-p cut per row
  int* cut_idx = nullptr;
  TopPScratch topp;             // the top-p passes' partials, histograms and state
  int nvchunk = 0;
  int* d_pos = nullptr;
  int* d_tok = nullptr;
  int* d_seq = nullptr;             // [64] sequence slot of each row of a slotted decode step
  std::vector<int> row_seq;         // slots of the decode step being enqueued
  // paged KV cache (qdec_kv_paged); page_size 0 = contiguous [seq][nkv][max_ctx]
  int page_size = 0, log2p = 0, n_pages = 0, table_w = 0;
  int* d_table = nullptr;           // [max_seqs][table_w] page of each position block
  std::vector<int> free_pages;      // pages no sequence holds (a stack)
  std::vector<std::vector<int>> seq_pages;  // pages each sequence holds, in position order
  StepParams* d_params = nullptr;   // per-step values read by replayed graphs
  hipStream_t cap_stream = nullptr; // capture stream for the decode graphs
  std::unordered_map<int, hipGraphExec_t> graphs;  // decode graph per batch size
  int* d_prompt = nullptr;
  int* err_host = nullptr;
  int* err_dev = nullptr;
  std::vector<int> kvlen;
  bool poisoned = false;
  int inject_fault = 0;  // qdec_debug_inject_fault: the next launch reports a synthetic error
  std::vector<void*> allocs;
  std::unordered_map<std::string, NameRef> names;
  bool timing = false;
  std::vector<KRec> krecs;
  std::vector<hipEvent_t> evpool;  // timing events, reused across timing passes
  size_t evnext = 0;
  hipStream_t last_stream = nullptr;

  const Mat& lm() const { return tied ? embd : out_w; }
  KvMap map() const { return KvMap{page_size ? d_table : nullptr, table_w, log2p, 0}; }
  // layer l's caches and row map
  float* lkc(int l) const { return kc + kv_off[l]; }
  float* lvc(int l) const { return vc + kv_off[l]; }
  KvMap lmap(int l) const {
    KvMap mp = map();
    mp.ring = kv_ring[l];
    return mp;
  }

  template <typename T>
  T* dalloc(size_t count) {
    void* p = nullptr;
    size_t bytes = std::max<size_t>(count * sizeof(T), 256);
    hipck(hipMalloc(&p, bytes), "hipMalloc");
    allocs.push_back(p);
    return reinterpret_cast<T*>(p);
  }
  void dfree(void* p) {
    auto it = std::find(allocs.begin(), allocs.end(), p);
    if (it != allocs.end()) {
      allocs.erase(it);
      (void)hipFree(p);
    }
  }
};

namespace {

hipEvent_t pool_event(qdec_model* m) {
  if (m->evnext == m->evpool.size()) {
    hipEvent_t e;
    hipck(hipEventCreateWithFlags(&e, hipEventDisableSystemFence), "hipEventCreate");
    m->evpool.push_back(e);
  }
  return m->evpool[m->evnext++];
}

// ------------------------------------------------------------ launch helpers

// Per-kernel timing: while timing is on, each launch is bracketed by two HIP
// events recorded on its stream.  Events come from a pool created up front
// (hipEventDisableSystemFence: no system-scope cache flush per record), so the
// host keeps ahead of the GPU and launches stay back to back.
hipEvent_t pool_event(qdec_model* m);

struct Timed {
  qdec_model* m;
  hipStream_t st;
  const char* cls;
  double bytes, flops;
  hipEvent_t a = nullptr, b = nullptr;
  Timed(qdec_model* mm, hipStream_t s, const char* c, double by, double fl) : m(mm), st(s), cls(c), bytes(by), flops(fl) {
    if (m && m->timing) {
      a = pool_event(m);
      b = pool_event(m);
      hipck(hipEventRecord(a, st), "hipEventRecord");
    }
  }
  ~Timed() noexcept(false) {
    if (std::uncaught_exceptions()) return;  // unwinding already: the first error is reported
    hipck(hipGetLastError(), cls);
    if (a) {
      hipck(hipEventRecord(b, st), "hipEventRecord");
      m->krecs.push_back(KRec{cls, a, b, bytes, flops});
    }
    if (m && m->inject_fault) {  // the launch above is enqueued: the failure path drains it
      m->inject_fault = 0;
      throw HipError{std::string("injected fault after enqueueing ") + cls + " (qdec_debug_inject_fault)"};
    }
  }
};

const char* gemv_class(int type) {
  switch (type) {
    case kQ4_0: return "gemv_q4_0";
    case kQ8_0: return "gemv_q8_0";
    case kQ4_K: return "gemv_q4_k";
    case kQ6_K: return "gemv_q6_k";
    default: return "gemv_f32";
  }
}
const char* gemm_class(int type) {
  switch (type) {
    case kQ4_0: return "gemm_q4_0";
    case kQ8_0: return "gemm_q8_0";
    case kQ4_K: return "gemm_q4_k";
    case kQ6_K: return "gemm_q6_k";
    default: return "gemm_f32";
  }
}

void gemv_type(int type, int M, int cls, int mode, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
  switch (type) {
    case kQ8_0: gemv_launch<kQ8_0>(M, cls, mode, grid, lds, st, a); break;
    case kQ4_0: gemv_launch<kQ4_0>(M, cls, mode, grid, lds, st, a); break;
    case kQ4_K: gemv_launch<kQ4_K>(M, cls, mode, grid, lds, st, a); break;
    case kQ6_K: gemv_launch<kQ6_K>(M, cls, mode, grid, lds, st, a); break;
    default: gemv_launch<kF32>(M, cls, mode, grid, lds, st, a); break;
  }
}

void gemm_type(int type, int kind, int mode, dim3 grid, hipStream_t st, const GemmArgs& a) {
  switch (type) {
    case kQ8_0: gemm_launch<kQ8_0>(kind, mode, grid, st, a); break;
    case kQ4_0: gemm_launch<kQ4_0>(kind, mode, grid, st, a); break;
    case kQ4_K: gemm_launch<kQ4_K>(kind, mode, grid, st, a); break;
    case kQ6_K: gemm_launch<kQ6_K>(kind, mode, grid, st, a); break;
    default: gemm_launch<kF32>(kind, mode, grid, st, a); break;
  }
}

// y[r][*] (op)= W x[r] for rows r < nrows, in launches of up to 16 rows that fit
// the LDS budget.  y_ind: read the output base from device memory instead.
// Residual prologue for sandwich norms: the input is x + RMSNorm(add) * add_w,
// written to out by the first workgroup (out may be null).
struct Resid {
  const float* add = nullptr;
  const float* add_w = nullptr;
  float* out = nullptr;
};

// Input from decode attention's accumulators (row r, element k: o[r][k] / l[r][k / hd]).
struct AccIn {
  const float* o = nullptr;
  const float* l = nullptr;
  int hd = 0;
  size_t stride = 0;  // floats between accumulator blocks
};

// amax: one input row whose greedy choice the epilogue also takes, into
// m->am_v / m->am_i (see argmax_final).  Returns the number of waves of the
// launch (the argmax partials).
int gemv(qdec_model* m, hipStream_t st, const Mat& w, const float* x, int ldx, const float* norm_w, float eps,
         float* y, int ldy, int nrows, int mode, float* const* y_ind = nullptr, Resid res = Resid{},
         const float* bias = nullptr, AccIn acc = AccIn{}, bool amax = false) {
  if (bias && mode != kModeStore) throw HipError{"gemv: a bias needs the store epilogue"};
  if (amax && (nrows != 1 || mode != kModeStore || acc.o))
    throw HipError{"gemv: the fused argmax takes one row and the store epilogue"};
  const int kp = w.nblk * 32;
  const size_t per_row = (size_t)kp * 4 + (nibble_layout(w.type) ? (size_t)w.nblk * 4 : 0);
  // rows per launch: a power of two (the kernel's M) whose staged inputs fit the LDS budget
  int cap = 16;
  while (cap > 1 && per_row * cap > kGemvLdsMax) cap /= 2;
  if (per_row > kGemvLdsMax) throw HipError{"gemv: input row too long for LDS"};
  const bool pair = mode == kModePairSilu || mode == kModePairGelu;
  int nwaves = 0;
  const bool plain = !res.add && !acc.o && !amax;
  for (int r0 = 0, mr = 0; r0 < nrows; r0 += mr) {
    // 5..16 rows of block-quantized weights: the matrix-core decode where it fits (no LDS
    // staging: up to 16 rows per launch at any row length)
    const int nout = pair ? w.rows / 2 : w.rows;
    const int ks = gemv_mfma_split(w.type, std::min(16, nrows - r0), mode, nout, w.nblk, norm_w != nullptr,
                                   res.add != nullptr, acc.o != nullptr, amax);
    mr = std::min(ks ? 16 : cap, nrows - r0);
    if (ks) {
      GemvArgs a{w.qs, w.d, w.rows, w.nblk, x ? x + (size_t)r0 * ldx : nullptr, ldx, norm_w, eps,
                 y ? y + (size_t)r0 * ldy : nullptr, ldy, mr, y_ind, (long)r0 * ldy,
                 nullptr, nullptr, nullptr, bias, w.sd};
      if (acc.o) {
        a.xd = acc.o + (size_t)r0 * ldx;
        a.xl = acc.l + (size_t)r0 * (ldx / acc.hd);
        a.xhd = acc.hd;
        a.xcstride = (long)acc.stride;
      }
      const double bytes =
          w.gguf_bytes + (double)mr * kp * (acc.o ? 4 * kAccCopies : 4) + (double)mr * nout * 4;
      Timed tm(m, st, gemv_class(w.type), bytes, 2.0 * mr * w.rows * (double)w.cols);
      gemv_type(w.type, 16, kGemvMfmaClass, mode, dim3((nout + 15) / 16, ks), 0, st, a);
      continue;
    }
    int M = 1;
    while (M < mr) M *= 2;
    const int cls = gemv_tile_class(pair, w.rows, M, kp, plain);
    const int R = class_rows(cls), NW = class_waves(cls);
    const int ngroups = pair ? w.rows / R : (w.rows + R - 1) / R;
    // waves stay resident and loop: at most four workgroups per CU, so the
    // input staging of each workgroup is amortised over many row groups;
    // enough waves that none finishes more than 64 outputs (each wave holds
    // its outputs in one register, a lane per output, until it is done)
    const int grid_cap = NW == 16 ? 256 : 1024;  // sixteen-wave workgroups: one per CU
    const int per_wave = 64 / (pair ? R / 2 : R);  // row groups per wave at most
    const int grid_min = (ngroups + per_wave * NW - 1) / (per_wave * NW);
    dim3 grid(std::max({1, grid_min, std::min((ngroups + NW - 1) / NW, grid_cap)}));
    GemvArgs a{w.qs, w.d, w.rows, w.nblk, x ? x + (size_t)r0 * ldx : nullptr, ldx, norm_w, eps,
               y ? y + (size_t)r0 * ldy : nullptr, ldy, mr, y_ind, (long)r0 * ldy,
               res.add ? res.add + (size_t)r0 * ldx : nullptr, res.add_w,
               res.out ? res.out + (size_t)r0 * ldx : nullptr, bias, w.sd};
    if (acc.o) {
      a.xd = acc.o + (size_t)r0 * ldx;
      a.xl = acc.l + (size_t)r0 * (ldx / acc.hd);
      a.xhd = acc.hd;
      a.xcstride = (long)acc.stride;
    }
    if (amax) {
      if ((int)grid.x * NW > m->am_n) throw HipError{"gemv: too many waves for the argmax partials"};
      a.amax_v = m->am_v;
      a.amax_i = m->am_i;
    }
    const size_t lds = per_row * M;
    const double bytes =
        w.gguf_bytes + (double)mr * kp * (acc.o ? 4 * kAccCopies : 4) + (double)mr * (pair ? w.rows / 2 : w.rows) * 4;
    Timed tm(m, st, gemv_class(w.type), bytes, 2.0 * mr * w.rows * (double)w.cols);
    gemv_type(w.type, M, cls, mode, grid, lds, st, a);
    nwaves = (int)grid.x * NW;
  }
  return nwaves;
}

// Prefill projection.  prec: QDEC_PREFILL_F32 (f32 operands, the default),
// QDEC_PREFILL_BF16X3 (exact three-term bf16 split of the activations) or
// QDEC_PREFILL_BF16 (activations rounded to bf16); -1 = the model's setting.
// F32 and K-quant weights always take the f32 kernels.
void gemm(qdec_model* m, hipStream_t st, const Mat& w, const float* x, int ldx, int T, float* y, int ldy, int mode,
          int prec = -1) {
  GemmArgs a{w.qs, w.d, w.rows, w.nblk, x, ldx, T, y, ldy, w.sd};
  dim3 grid((w.rows + 127) / 128, (T + 63) / 64);
  const bool pair = mode == kModePairSilu || mode == kModePairGelu;
  if (prec < 0) prec = m ? m->prefill_prec : QDEC_PREFILL_F32;
  // few 64 x 128 tiles for the CUs: the f32 K-split tile below is faster there
  const bool few = (size_t)grid.x * grid.y < 512 && w.nblk >= 8;
  // the bf16 tile keeps the wide shape down to one 64 x 128 tile per CU (its
  // per-CU rate is many times the f32 tile's); below that the f32 K-split wins
  const bool few_bf16 = !pair && (size_t)grid.x * grid.y < 256 && w.nblk >= 8;
  if (prec != QDEC_PREFILL_F32 && (w.type == kQ8_0 || w.type == kQ4_0) && !few_bf16) {
    const int nt = prec == QDEC_PREFILL_BF16X3 ? 3 : 1;
    const double bytes = w.gguf_bytes + (double)T * w.nblk * 32 * 4 + (double)T * (pair ? w.rows / 2 : w.rows) * 4;
    // flops: the algorithmic 2 T N K (each term's products are extra MFMA work)
    Timed tm(m, st, nt == 3 ? (w.type == kQ8_0 ? "gemm_bf16x3_q8_0" : "gemm_bf16x3_q4_0")
                            : (w.type == kQ8_0 ? "gemm_bf16_q8_0" : "gemm_bf16_q4_0"),
             bytes, 2.0 * T * (double)w.rows * w.cols);
    gemm_type(w.type, nt == 3 ? kGemmBf16x3 : kGemmBf16, mode, grid, st, a);
    return;
  }
  // few 64 x 128 tiles for the CUs: switch to the K-split 32 x 64 tile, with
  // eight waves when even its grid gives a CU about one workgroup
  if (few) {
    dim3 g2((w.rows + 63) / 64, (T + 31) / 32);
    const bool eight = (size_t)g2.x * g2.y < 512 && w.nblk >= 16;
    const double bytes = w.gguf_bytes + (double)T * w.nblk * 32 * 4 + (double)T * (pair ? w.rows / 2 : w.rows) * 4;
    Timed tm(m, st, gemm_class(w.type), bytes, 2.0 * T * (double)w.rows * w.cols);
    gemm_type(w.type, eight ? kGemmKSplit8 : kGemmKSplit, mode, g2, st, a);
    return;
  }
  const double bytes = w.gguf_bytes + (double)T * w.nblk * 32 * 4 + (double)T * (pair ? w.rows / 2 : w.rows) * 4;
  Timed tm(m, st, gemm_class(w.type), bytes, 2.0 * T * (double)w.rows * w.cols);
  gemm_type(w.type, kGemmWide, mode, grid, st, a);
}

void rmsnorm_rows(qdec_model* m, hipStream_t st, const float* x, int ldx, const float* w, int n, float* out, int ldo,
                  int rows, int add) {
  NormArgs a{x, ldx, w, m ? m->cfg.rms_eps : 0.f, n, out, ldo, add};
  Timed tm(m, st, "rmsnorm", (double)rows * n * (add ? 12 : 8), 0);
  qlaunch(rmsnorm_kernel, rows, 256, 0, st, a);
}

template <int HD, bool PAGED>
void attn_decode_hd(int G, dim3 grid, hipStream_t st, const AttnDecodeArgs& a) {
  switch (G) {
    case 1: qlaunch(attn_decode_kernel<HD, 1, PAGED>, grid, 256, 0, st, a); break;
    case 2: qlaunch(attn_decode_kernel<HD, 2, PAGED>, grid, 256, 0, st, a); break;
    case 4: qlaunch(attn_decode_kernel<HD, 4, PAGED>, grid, 256, 0, st, a); break;
    default: throw HipError{"attention: query heads per KV head per workgroup must be 1, 2 or 4"};
  }
}

int layer_window(const qdec_model* m, int l) { return m->layers[l].global ? 0 : m->cfg.window; }

// Ring of a sliding-window layer in the contiguous cache: R = the power of two
// >= window + ws_T - 1 (ws_T: the rows of one prefill pass), at least 64, used
// when it at most halves the layer (R <= max_ctx / 2).  A prefill pass appends
// ws_T positions at most, and its queries need the window - 1 positions before
// them: all of them fit in the ring, so the pass appends and attends as with
// the full cache.
int ring_log2(const qdec_model* m, int l) {
  const int w = layer_window(m, l);
  if (!m->ring_on || m->page_size || w <= 0) return 0;
  int lg = 6;
  while ((int64_t)1 << lg < (int64_t)w + m->ws_T - 1) ++lg;
  return ((int64_t)2 << lg) <= m->max_ctx ? lg : 0;
}

// Lay out and clear the contiguous caches: each layer [max_seqs][nkv][positions][hd]
// with max_ctx positions, or its ring.
void layout_contiguous(qdec_model* m, hipStream_t st) {
  const qdec_config& c = m->cfg;
  m->kv_off.assign(c.n_layer, 0);
  m->kv_ring.assign(c.n_layer, 0);
  size_t total = 0;
  m->kv_layer = 0;
  for (int l = 0; l < c.n_layer; ++l) {
    m->kv_ring[l] = ring_log2(m, l);
    const size_t pos = m->kv_ring[l] ? (size_t)1 << m->kv_ring[l] : (size_t)m->max_ctx;
    const size_t layer = (size_t)m->max_seqs * c.n_head_kv * pos * c.head_dim;
    m->kv_off[l] = total;
    total += layer;
    m->kv_layer = std::max(m->kv_layer, layer);
  }
  m->kc = m->dalloc<float>(total);
  m->vc = m->dalloc<float>(total);
  // rows past a sequence's length are read (and masked) by decode attention:
  // start from finite values
  hipck(hipMemsetAsync(m->kc, 0, total * 4, st), "memset");
  hipck(hipMemsetAsync(m->vc, 0, total * 4, st), "memset");
}

// slotted: row b serves sequence d_seq[b] (continuous batching), else b.
void attention_decode(qdec_model* m, hipStream_t st, int l, int B, bool slotted) {
  const qdec_config& c = m->cfg;
  const Layer& L = m->layers[l];
  const int hd = c.head_dim, G = c.n_head / c.n_head_kv;
  const float scale_log2 = (float)(1.0 / std::sqrt((double)hd) * 1.4426950408889634);
  AttnDecodeArgs a{m->qkv, m->nqkv, m->lkc(l), m->lvc(l), m->max_ctx, m->d_pos,
                   c.n_head, c.n_head_kv, layer_window(m, l), m->chunk, m->nchunk, L.q_norm, L.k_norm, c.rms_eps,
                   m->rope_cur + (L.global ? 0 : (size_t)m->max_seqs * (hd / 2)), scale_log2,
                   m->acc + (size_t)(l % 2) * kAccCopies * m->acc_blk,
                   m->acc + (size_t)((l + 1) % 2) * kAccCopies * m->acc_blk, m->max_seqs, m->err_dev,
                   slotted ? m->d_seq : nullptr, m->lmap(l), G == 8 ? 2 : 1};
  double kvbytes = 0;
  for (int s = 0; s < B; ++s) {
    int p = m->kvlen[(size_t)s < m->row_seq.size() ? m->row_seq[s] : s];
    int lo = a.window > 0 ? std::max(0, p - a.window + 1) : 0;
    kvbytes += (double)(p - lo + 1) * c.n_head_kv * hd * 8;
  }
  {
    Timed tm(m, st, "attn_decode", kvbytes + (double)B * m->nqkv * 4, 4.0 * kvbytes / 8 * G);
    dim3 grid(m->nchunk, c.n_head_kv * a.gsplit, B);
    const bool pg = m->page_size > 0;
    const int Gw = G / a.gsplit;  // query heads per workgroup
    if (hd == 64) pg ? attn_decode_hd<64, true>(Gw, grid, st, a) : attn_decode_hd<64, false>(Gw, grid, st, a);
    else if (hd == 128) pg ? attn_decode_hd<128, true>(Gw, grid, st, a) : attn_decode_hd<128, false>(Gw, grid, st, a);
    else pg ? attn_decode_hd<256, true>(Gw, grid, st, a) : attn_decode_hd<256, false>(Gw, grid, st, a);
  }
}

void attention_prefill(qdec_model* m, hipStream_t st, int l, int seq, int T, int pos0) {
  const qdec_config& c = m->cfg;
  const int hd = c.head_dim;
  AttnPrefillArgs a{m->q, m->lkc(l), m->lvc(l), m->max_ctx, T, pos0, c.n_head, c.n_head_kv, layer_window(m, l),
                    (float)(1.0 / std::sqrt((double)hd) * 1.4426950408889634), m->a, seq, m->lmap(l)};
  double pairs = 0;
  for (int t = 0; t < T; ++t) {
    int p = pos0 + t, lo = a.window > 0 ? std::max(0, p - a.window + 1) : 0;
    pairs += p - lo + 1;
  }
  Timed tm(m, st, "attn_prefill", (double)T * c.n_head * hd * 8 + (double)(pos0 + T) * c.n_head_kv * hd * 8,
           4.0 * hd * c.n_head * pairs);
  // the matrix-core kernels (32 queries per workgroup): head_dim 64 and 128
  // whole-head per wave, 256 split over the four waves.  They index cache rows
  // in 32 bits: the loader and qdec_kv_paged keep a layer below 2^31 rows.
  if (m->kv_layer / hd >= (size_t)INT32_MAX) throw HipError{"prefill attention: cache layer of 2^31 rows or more"};
  const int nqt = (T + 31) / 32;
  if (hd == 64) qlaunch(attn_prefill_mfma_kernel<64>, dim3(nqt * c.n_head), 256, 0, st, a);
  else if (hd == 128) qlaunch(attn_prefill_mfma_kernel<128>, dim3(nqt * c.n_head), 256, 0, st, a);
  else qlaunch(attn_prefill_dsplit_kernel<256>, dim3(nqt * c.n_head), 256, 0, st, a);
}

void rope_kv(qdec_model* m, hipStream_t st, int l, int n, int seq0, int pos0, const int* dpos) {
  const qdec_config& c = m->cfg;
  const Layer& L = m->layers[l];
  RopeArgs a{m->qkv, m->nqkv, m->q, m->lkc(l), m->lvc(l), m->max_ctx, c.n_head, c.n_head_kv, c.head_dim,
             L.q_norm, L.k_norm, c.rms_eps, L.global ? m->rope_g : m->rope_l, seq0, pos0, dpos, L.qkv_bias,
             m->lmap(l)};
  Timed tm(m, st, "rope_kv", (double)n * m->nqkv * 8, 0);
  qlaunch(rope_kv_kernel, dim3(n, (c.n_head + 2 * c.n_head_kv + 3) / 4), 256, 0, st, a);
}

void embed(qdec_model* m, hipStream_t st, const int* d_tokens, int n, float* out) {
  const qdec_config& c = m->cfg;
  EmbedArgs a{WView{m->embd.qs, m->embd.d, m->embd.type, m->embd.nblk, m->embd.sd}, c.hidden, c.vocab, n, d_tokens, out,
              c.hidden, m->err_dev};
  Timed tm(m, st, "embed", (double)n * (m->embd.gguf_bytes / m->embd.rows + c.hidden * 4), 0);
  switch (m->embd.type) {
    case kQ8_0: qlaunch(embed_kernel<kQ8_0>, n, 256, 0, st, a); break;
    case kQ4_0: qlaunch(embed_kernel<kQ4_0>, n, 256, 0, st, a); break;
    case kQ4_K: qlaunch(embed_kernel<kQ4_K>, n, 256, 0, st, a); break;
    case kQ6_K: qlaunch(embed_kernel<kQ6_K>, n, 256, 0, st, a); break;
    default: qlaunch(embed_kernel<kF32>, n, 256, 0, st, a); break;
  }
}

// The top-p cut of rows x vocab logits: the seven passes of topp_pass_kernel.
void topp_cut(hipStream_t st, TopPArgs t) {
  for (int pass = 0; pass <= 6; ++pass) {
    t.pass = pass;
    qlaunch(topp_pass_kernel, pass < 6 ? dim3(kTopPChunks, t.rows) : dim3(1, t.rows), 256, 0, st, t);
  }
}

void sample(qdec_model* m, hipStream_t st, const float* logits, int ld, int rows, float temp, uint64_t seed,
            uint64_t step, int* out, int* out2, const StepParams* sp = nullptr, bool topp = false,
            const int* seq = nullptr) {
  const int V = m->cfg.vocab;
  SampleArgs a{logits, ld, V, rows, temp, seed, step, m->s_v, m->s_i, m->nvchunk, out, out2, sp,
               topp ? m->cut_key : nullptr, topp ? m->cut_idx : nullptr, seq};
  if (topp) {
    TopPArgs t{logits, ld, V, rows, temp, 1.f, m->cut_key, m->cut_idx, sp, m->topp.pmax, m->topp.pbad,
               m->topp.hist, m->topp.state, 0};
    Timed tm(m, st, "topp_cut", (double)rows * V * 4 * 6, 0);
    topp_cut(st, t);
  }
  {
    Timed tm(m, st, "sample", (double)rows * V * 4, 0);
    qlaunch(sample_stage1_kernel, dim3(m->nvchunk, rows), 256, 0, st, a);
  }
  Timed tm(m, st, "sample_final", (double)rows * m->nvchunk * 8, 0);
  qlaunch(sample_stage2_kernel, rows, 64, 0, st, a);
}

// The greedy token of one row from the LM head's fused per-wave choices
// (gemv with amax): one workgroup reduces the nwaves partials.  out, or the
// step parameters' token buffer when sp is given.
void argmax_final(qdec_model* m, hipStream_t st, int nwaves, int* out, const StepParams* sp = nullptr) {
  if (nwaves > m->am_n) throw HipError{"argmax_final: too many partials"};
  SampleArgs a{nullptr, 0, m->cfg.vocab, 1, 0.f, 0, 0, m->am_v, m->am_i, nwaves, out, nullptr, sp,
               nullptr, nullptr, nullptr};
  Timed tm(m, st, "argmax_final", (double)nwaves * 8, 0);
  qlaunch(argmax_waves_kernel, 1, 1024, 0, st, a);
}

// q|k|v projection of decode rows into m->qkv (RMSNorm prologue, optional
// residual prologue, bias epilogue): one launch over the fused rows, or three
// when q, k and v have different types.  With a residual prologue each of the
// three launches writes the same new residual row.
void qkv_gemv(qdec_model* m, hipStream_t st, const Layer& L, const float* x, int n, Resid res) {
  const qdec_config& c = m->cfg;
  if (!L.qkv_split) {
    gemv(m, st, L.qkv, x, c.hidden, L.attn_norm, c.rms_eps, m->qkv, m->nqkv, n, kModeStore, nullptr, res, L.qkv_bias);
    return;
  }
  const int off[3] = {0, m->qd, m->qd + m->kd};
  for (int j = 0; j < 3; ++j)
    gemv(m, st, L.qkv_part[j], x, c.hidden, L.attn_norm, c.rms_eps, m->qkv + off[j], m->nqkv, n, kModeStore, nullptr,
         res, L.qkv_bias ? L.qkv_bias + off[j] : nullptr);
}

// The blocks over n tokens of one sequence (prefill) or one token of each of n
// sequences (decode, dpos != null); the residual stream is m->x.
void blocks(qdec_model* m, hipStream_t st, int n, int seq, int pos0, const int* dpos, bool slotted = false) {
  const qdec_config& c = m->cfg;
  const int H = c.hidden;
  const bool dec = dpos != nullptr;
  const int act_mode = c.act == QDEC_ACT_GELU_TANH ? kModePairGelu : kModePairSilu;
  // Decode with sandwich norms: each post-norm and its residual add run in the
  // prologue of the next GEMV (Resid), which writes the new residual row to the
  // other of two buffers (the kernel's other workgroups still read the old
  // one): R_l in x, R_l + post-attention term in x2, the next R in x again.
  const bool fuse = dec && c.sandwich_norm;
  for (int l = 0; l < c.n_layer; ++l) {
    const Layer& L = m->layers[l];
    // attention sublayer
    if (fuse && l > 0) {
      qkv_gemv(m, st, L, m->x2, n, Resid{m->y, m->layers[l - 1].post_ffw, m->x});
    } else if (dec) {
      qkv_gemv(m, st, L, m->x, n, Resid{});
    } else {
      rmsnorm_rows(m, st, m->x, H, L.attn_norm, H, m->h, H, n, 0);
      if (!L.qkv_split) {
        gemm(m, st, L.qkv, m->h, H, n, m->qkv, m->nqkv, kModeStore);
      } else {
        const int off[3] = {0, m->qd, m->qd + m->kd};
        for (int j = 0; j < 3; ++j) gemm(m, st, L.qkv_part[j], m->h, H, n, m->qkv + off[j], m->nqkv, kModeStore);
      }
    }
    if (dec) {
      attention_decode(m, st, l, n, slotted);  // QK-norm, RoPE and the KV append run inside
    } else {
      // a ring holds the window plus a whole pass (ring_log2)
      if (m->kv_ring[l] && n > (1 << m->kv_ring[l]) - layer_window(m, l) + 1)
        throw HipError{"prefill pass longer than the window layer's ring"};
      rope_kv(m, st, l, n, seq, pos0, nullptr);
      attention_prefill(m, st, l, seq, n, pos0);
    }
    // decode: the O projection's input is attention's merge, o / l from the
    // accumulators of this layer's parity
    const float* acc_o = m->acc + (size_t)(l % 2) * kAccCopies * m->acc_blk;
    const AccIn acc{acc_o, acc_o + (size_t)m->max_seqs * m->qd, c.head_dim, m->acc_blk};
    if (fuse) {
      gemv(m, st, L.o, nullptr, m->qd, nullptr, 0.f, m->y, H, n, kModeStore, nullptr, Resid{}, nullptr, acc);
    } else if (c.sandwich_norm) {
      gemm(m, st, L.o, m->a, m->qd, n, m->y, H, kModeStore);
      rmsnorm_rows(m, st, m->y, H, L.post_attn, H, m->x, H, n, 1);
    } else {
      if (dec) gemv(m, st, L.o, nullptr, m->qd, nullptr, 0.f, m->x, H, n, kModeAdd, nullptr, Resid{}, nullptr, acc);
      else gemm(m, st, L.o, m->a, m->qd, n, m->x, H, kModeAdd);
    }
    // feed-forward sublayer
    if (fuse) {
      gemv(m, st, L.gu, m->x, H, L.ffn_norm, c.rms_eps, m->m, m->Fp, n, act_mode, nullptr,
           Resid{m->y, L.post_attn, m->x2});
    } else if (dec) {
      gemv(m, st, L.gu, m->x, H, L.ffn_norm, c.rms_eps, m->m, m->Fp, n, act_mode);
    } else {
      rmsnorm_rows(m, st, m->x, H, L.ffn_norm, H, m->h, H, n, 0);
      gemm(m, st, L.gu, m->h, H, n, m->m, m->Fp, act_mode);
    }
    if (fuse) {
      gemv(m, st, L.down, m->m, m->Fp, nullptr, 0.f, m->y, H, n, kModeStore);
    } else if (c.sandwich_norm) {
      gemm(m, st, L.down, m->m, m->Fp, n, m->y, H, kModeStore);
      rmsnorm_rows(m, st, m->y, H, L.post_ffw, H, m->x, H, n, 1);
    } else {
      if (dec) gemv(m, st, L.down, m->m, m->Fp, nullptr, 0.f, m->x, H, n, kModeAdd);
      else gemm(m, st, L.down, m->m, m->Fp, n, m->x, H, kModeAdd);
    }
  }
}

// One decode step for sequences 0..n-1 reading tokens, positions and the
// step's parameters from device memory (so it can be captured and replayed).
// greedy1: one row at temperature 0, whose token the LM head's epilogue picks
void decode_body(qdec_model* m, hipStream_t st, int n, bool topp, bool slotted, bool greedy1) {
  const qdec_config& c = m->cfg;
  embed(m, st, m->d_tok, n, m->x);
  blocks(m, st, n, 0, 0, m->d_pos, slotted);
  int nw;
  if (c.sandwich_norm)  // the last post-FFN norm and residual add run in the head's prologue
    nw = gemv(m, st, m->lm(), m->x2, c.hidden, m->output_norm, c.rms_eps, nullptr, c.vocab, n, kModeStore,
              &m->d_params->logits, Resid{m->y, m->layers[c.n_layer - 1].post_ffw, nullptr}, nullptr,
              AccIn{}, greedy1);
  else
    nw = gemv(m, st, m->lm(), m->x, c.hidden, m->output_norm, c.rms_eps, nullptr, c.vocab, n, kModeStore,
              &m->d_params->logits, Resid{}, nullptr, AccIn{}, greedy1);
  if (greedy1) argmax_final(m, st, nw, nullptr, m->d_params);
  else sample(m, st, nullptr, c.vocab, n, 0.f, 0, 0, nullptr, nullptr, m->d_params, topp, slotted ? m->d_seq : nullptr);
}

// ------------------------------------------------------------ error handling
void drain(hipStream_t st) {
  hipEvent_t ev;
  if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return;
  if (hipEventRecord(ev, st) == hipSuccess) {
    auto t0 = std::chrono::steady_clock::now();
    while (hipEventQuery(ev) == hipErrorNotReady) {
      if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(30)) {
        g_err += " (stream still busy after the 30 s wait)";
        break;
      }
      std::this_thread::sleep_for(std::chrono::microseconds(200));
    }
  }
  (void)hipEventDestroy(ev);
}

int fail_internal(qdec_model* m, hipStream_t st, const std::string& msg) {
  set_err("internal: %s", msg.c_str());
  (void)hipGetLastError();
  drain(st);
  if (m) m->poisoned = true;
  return QDEC_INTERNAL;
}

int check_usable(qdec_model* m) {
  if (!m) {
    set_err("model handle is NULL");
    return QDEC_REFUSED;
  }
  if (m->poisoned) {
    set_err("poisoned: an earlier GPU failure latched this handle; free it and load again");
    return QDEC_REFUSED;
  }
  if (m->err_host) {
    const int e = __atomic_load_n(m->err_host, __ATOMIC_ACQUIRE);
    if (e) {
      m->poisoned = true;
      if (e == 2)
        set_err("internal: decode attention met scores 100 or more log2 units above the new token's own "
                "score (or NaN scores); handle poisoned");
      else
        set_err("internal: a device-resident token id was outside [0, vocab) (clamped); handle poisoned");
      return QDEC_INTERNAL;
    }
  }
  return QDEC_OK;
}

// ------------------------------------------------------------ loading
struct Expect {
  std::string name;
  int64_t rows, cols;
  bool matrix;  // quantized allowed
  bool required;
};

std::vector<Expect> expected_tensors(const qdec_config& c) {
  std::vector<Expect> e;
  const int64_t H = c.hidden, hd = c.head_dim, qd = (int64_t)c.n_head * hd, kd = (int64_t)c.n_head_kv * hd;
  e.push_back({"token_embd.weight", c.vocab, H, true, true});
  for (int i = 0; i < c.n_layer; ++i) {
    std::string p = "blk." + std::to_string(i) + ".";
    e.push_back({p + "attn_norm.weight", 1, H, false, true});
    e.push_back({p + "attn_q.weight", qd, H, true, true});
    e.push_back({p + "attn_k.weight", kd, H, true, true});
    e.push_back({p + "attn_v.weight", kd, H, true, true});
    if (c.qkv_bias) {
      e.push_back({p + "attn_q.bias", 1, qd, false, true});
      e.push_back({p + "attn_k.bias", 1, kd, false, true});
      e.push_back({p + "attn_v.bias", 1, kd, false, true});
    }
    if (c.qk_norm) {
      e.push_back({p + "attn_q_norm.weight", 1, hd, false, true});
      e.push_back({p + "attn_k_norm.weight", 1, hd, false, true});
    }
    e.push_back({p + "attn_output.weight", H, qd, true, true});
    if (c.sandwich_norm) e.push_back({p + "post_attention_norm.weight", 1, H, false, true});
    e.push_back({p + "ffn_norm.weight", 1, H, false, true});
    e.push_back({p + "ffn_gate.weight", c.ffn, H, true, true});
    e.push_back({p + "ffn_up.weight", c.ffn, H, true, true});
    e.push_back({p + "ffn_down.weight", H, c.ffn, true, true});
    if (c.sandwich_norm) e.push_back({p + "post_ffw_norm.weight", 1, H, false, true});
  }
  e.push_back({"output_norm.weight", 1, H, false, true});
  e.push_back({"output.weight", c.vocab, H, true, false});
  return e;
}

bool scales_finite(const qdec_tensor& t) {
  auto finite = [](const uint8_t* p) { return ((p[1] >> 2) & 0x1f) != 0x1f; };
  const uint8_t* b = static_cast<const uint8_t*>(t.host_data);
  if (is_kquant(t.type)) {
    const int64_t nb = t.rows * (t.cols / 256), bb = super_bytes(t.type);
    for (int64_t i = 0; i < nb; ++i) {
      const uint8_t* sb = b + i * bb;
      if (t.type == kQ4_K ? !(finite(sb) && finite(sb + 2)) : !finite(sb + 208)) return false;
    }
    return true;
  }
  if (!is_quant(t.type)) return true;
  const int64_t nb = t.rows * nblocks(t.cols), bb = blk_bytes(t.type);
  for (int64_t i = 0; i < nb; ++i)
    if (!finite(b + i * bb)) return false;
  return true;
}

// Repack GGUF rows [src_rows][blocks] into (quants, scales) at device row dst_row
// of a host staging buffer of the fused matrix.
// K-quant super-blocks are repacked into the 32-value layouts of the legacy
// types (GGUF's public K-quant layouts), keeping the scales as the file has
// them, unpacked to whole bytes:
//   Q4_K (fp16 d, fp16 dmin, 12 bytes of eight 6-bit (scale, min) pairs, 128
//   quant bytes whose low / high nibbles hold sub-blocks 2c / 2c + 1) -> per
//   sub-block the Q4_0 nibble order and a u16 sc | m << 8; per super-block a
//   u32 d | dmin << 16;
//   Q6_K (128 low-nibble bytes, 64 bytes of 2-bit high parts, 16 int8 scales,
//   fp16 d) -> int8 q - 32 per value, the int8 scale per 16 values, and per
//   super-block a u32 holding d.
// The kernels form d * sc, dmin * m, d * scale in f32 (exact: at most 11 + 8
// significant bits).
struct Stage {
  int type;
  int64_t rows, nblk;
  std::vector<uint8_t> qs;
  std::vector<uint16_t> d;
  std::vector<uint8_t> ks;   // K-quants: 2 bytes per 32-value block (Q4_K sc, m; Q6_K two int8 scales)
  std::vector<uint32_t> sd;  // K-quants: one word per 256-value super-block
  Stage(int t, int64_t r, int64_t nb) : type(t), rows(r), nblk(nb) {
    const bool nib = t == kQ4_0 || t == kQ4_K, i8 = t == kQ8_0 || t == kQ6_K;
    qs.assign((size_t)(nib ? r * nb * 16 : i8 ? r * nb * 32 : r * nb * 32 * 4), 0);
    if (is_quant(t)) d.assign((size_t)(r * nb), 0);
    if (is_kquant(t)) {
      ks.assign((size_t)(2 * r * nb), 0);
      sd.assign((size_t)(r * (nb / 8)), 0);
    }
  }
  void put_q4_k(int64_t dst_row, const uint8_t* src, int64_t nsb) {
    for (int64_t sbi = 0; sbi < nsb; ++sbi) {
      const uint8_t* sb = src + sbi * 144;
      sd[(size_t)(dst_row * (nblk / 8) + sbi)] =
          (uint32_t)(sb[0] | sb[1] << 8) | (uint32_t)(sb[2] | sb[3] << 8) << 16;
      const uint8_t* sc = sb + 4;
      const uint8_t* q = sb + 16;
      for (int j = 0; j < 8; ++j) {
        const int scale = j < 4 ? sc[j] & 63 : (sc[j + 4] & 15) | ((sc[j - 4] >> 6) << 4);
        const int mn = j < 4 ? sc[j + 4] & 63 : (sc[j + 4] >> 4) | ((sc[j] >> 6) << 4);
        const int64_t b = dst_row * nblk + sbi * 8 + j;
        ks[(size_t)(2 * b)] = (uint8_t)scale;
        ks[(size_t)(2 * b + 1)] = (uint8_t)mn;
        const uint8_t* qc = q + 32 * (j / 2);
        const int sh = 4 * (j & 1);
        for (int i = 0; i < 16; ++i) {
          const uint8_t lo = (qc[i] >> sh) & 15, hi = (qc[i + 16] >> sh) & 15;
          qs[(size_t)(b * 16 + i)] = (uint8_t)(lo | hi << 4);
        }
      }
    }
  }
  void put_q6_k(int64_t dst_row, const uint8_t* src, int64_t nsb) {
    int8_t* out = reinterpret_cast<int8_t*>(qs.data()) + dst_row * nblk * 32;
    for (int64_t sbi = 0; sbi < nsb; ++sbi) {
      const uint8_t* sb = src + sbi * 210;
      sd[(size_t)(dst_row * (nblk / 8) + sbi)] = (uint32_t)(sb[208] | sb[209] << 8);
      for (int h = 0; h < 2; ++h) {
        const uint8_t* ql = sb + 64 * h;
        const uint8_t* qh = sb + 128 + 32 * h;
        int8_t* o = out + sbi * 256 + 128 * h;
        for (int l = 0; l < 32; ++l) {
          o[l] = (int8_t)(((ql[l] & 15) | ((qh[l] & 3) << 4)) - 32);
          o[l + 32] = (int8_t)(((ql[l + 32] & 15) | (((qh[l] >> 2) & 3) << 4)) - 32);
          o[l + 64] = (int8_t)(((ql[l] >> 4) | (((qh[l] >> 4) & 3) << 4)) - 32);
          o[l + 96] = (int8_t)(((ql[l + 32] >> 4) | ((qh[l] >> 6) << 4)) - 32);
        }
      }
      for (int g = 0; g < 16; ++g) ks[(size_t)(dst_row * 2 * nblk + sbi * 16 + g)] = sb[192 + g];
    }
  }
  void put_row(int64_t dst_row, const qdec_tensor& t, int64_t src_row) {
    const uint8_t* src = static_cast<const uint8_t*>(t.host_data);
    const int64_t nb = nblocks(t.cols);
    if (is_kquant(type)) {
      const int64_t nsb = t.cols / 256;
      const uint8_t* row = src + src_row * nsb * super_bytes(type);
      if (type == kQ4_K) put_q4_k(dst_row, row, nsb);
      else put_q6_k(dst_row, row, nsb);
      return;
    }
    if (type == kF32) {
      std::memcpy(&qs[(size_t)dst_row * nblk * 32 * 4], src + src_row * t.cols * 4, (size_t)t.cols * 4);
      return;
    }
    const int64_t bb = blk_bytes(type), payload = bb - 2;
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* blk = src + (src_row * nb + b) * bb;
      d[(size_t)(dst_row * nblk + b)] = (uint16_t)blk[0] | ((uint16_t)blk[1] << 8);
      std::memcpy(&qs[(size_t)((dst_row * nblk + b) * payload)], blk + 2, (size_t)payload);
    }
  }
};

Mat upload(qdec_model* m, const Stage& s, int rows, int cols, double gguf_bytes, hipStream_t st) {
  Mat w;
  w.type = s.type;
  w.rows = rows;
  w.cols = cols;
  w.nblk = (int)s.nblk;
  w.gguf_bytes = gguf_bytes;
  w.qs = m->dalloc<uint8_t>(s.qs.size());
  hipck(hipMemcpyAsync(w.qs, s.qs.data(), s.qs.size(), hipMemcpyHostToDevice, st), "upload");
  if (is_quant(s.type)) {
    w.d = m->dalloc<uint16_t>(s.d.size());
    hipck(hipMemcpyAsync(w.d, s.d.data(), s.d.size() * 2, hipMemcpyHostToDevice, st), "upload");
  }
  if (is_kquant(s.type)) {  // per-sub-block scale words (through d) and super-block scales
    w.d = m->dalloc<uint16_t>(s.ks.size() / 2);
    hipck(hipMemcpyAsync(w.d, s.ks.data(), s.ks.size(), hipMemcpyHostToDevice, st), "upload");
    w.sd = m->dalloc<uint32_t>(s.sd.size());
    hipck(hipMemcpyAsync(w.sd, s.sd.data(), s.sd.size() * 4, hipMemcpyHostToDevice, st), "upload");
  }
  hipck(hipStreamSynchronize(st), "upload sync");
  return w;
}

float* upload_vec(qdec_model* m, const qdec_tensor& t, hipStream_t st) {
  float* p = m->dalloc<float>((size_t)t.cols);
  hipck(hipMemcpyAsync(p, t.host_data, (size_t)t.cols * 4, hipMemcpyHostToDevice, st), "upload");
  return p;
}

void free_model(qdec_model* m) {
  for (auto& g : m->graphs)
    if (g.second) (void)hipGraphExecDestroy(g.second);
  m->graphs.clear();
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  for (void* p : m->allocs) (void)hipFree(p);
  m->allocs.clear();
  for (hipEvent_t e : m->evpool) (void)hipEventDestroy(e);
  if (m->err_host) (void)hipHostFree(m->err_host);
  delete m;
}

int load(const qdec_config* cfgp, const qdec_tensor* ts, int32_t n, int32_t max_seqs, int32_t max_ctx,
         hipStream_t st, qdec_model** out) {
  if (!cfgp || !out) {
    set_err("cfg and out must not be NULL");
    return QDEC_REFUSED;
  }
  *out = nullptr;
  const qdec_config c = *cfgp;
  if (c.n_layer <= 0 || c.hidden <= 0 || c.n_head <= 0 || c.n_head_kv <= 0 || c.head_dim <= 0 || c.ffn <= 0 ||
      c.vocab <= 0) {
    set_err("config: every dimension must be positive");
    return QDEC_REFUSED;
  }
  if (c.hidden % 32) { set_err("config: hidden (%d) must be a multiple of 32", c.hidden); return QDEC_REFUSED; }
  if (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256) {
    set_err("config: head_dim %d unsupported (64, 128 or 256)", c.head_dim);
    return QDEC_REFUSED;
  }
  if (c.n_head % c.n_head_kv) { set_err("config: n_head must be a multiple of n_head_kv"); return QDEC_REFUSED; }
  const int G = c.n_head / c.n_head_kv;
  if (!(G == 1 || G == 2 || G == 4 || (G == 8 && c.head_dim == 128))) {
    set_err("config: query heads per KV head = %d unsupported (1, 2, 4; 8 with head_dim 128)", G);
    return QDEC_REFUSED;
  }
  if (c.act != QDEC_ACT_SILU && c.act != QDEC_ACT_GELU_TANH) { set_err("config: act must be 0 or 1"); return QDEC_REFUSED; }
  if (c.window < 0 || (c.window > 0 && c.window_period <= 0)) {
    set_err("config: window >= 0, and window_period >= 1 when window > 0");
    return QDEC_REFUSED;
  }
  if (!(c.rms_eps >= 0.f) || !std::isfinite(c.rms_eps) || !(c.rope_theta > 0.f) ||
      (c.window > 0 && !(c.rope_theta_local > 0.f))) {
    set_err("config: rms_eps must be finite and >= 0, rope thetas > 0");
    return QDEC_REFUSED;
  }
  if (max_seqs < 1 || max_seqs > 64) { set_err("max_seqs must be in [1, 64], got %d", max_seqs); return QDEC_REFUSED; }
  if (max_ctx < 1) { set_err("max_ctx must be >= 1"); return QDEC_REFUSED; }
  if ((int64_t)max_seqs * c.n_head_kv * max_ctx >= INT32_MAX) {
    set_err("max_seqs x n_head_kv x max_ctx = %lld cache rows per layer; the kernels index fewer than 2^31",
            (long long)max_seqs * c.n_head_kv * max_ctx);
    return QDEC_REFUSED;
  }
  if (n < 0 || (n > 0 && !ts)) { set_err("tensors: NULL array or negative count"); return QDEC_REFUSED; }

  // validate every tensor before allocating anything
  std::vector<Expect> exp = expected_tensors(c);
  std::unordered_map<std::string, const Expect*> byname;
  for (auto& e : exp) byname[e.name] = &e;
  std::unordered_map<std::string, const qdec_tensor*> got;
  for (int i = 0; i < n; ++i) {
    const qdec_tensor& t = ts[i];
    if (!t.name) { set_err("tensor %d: NULL name", i); return QDEC_REFUSED; }
    auto it = byname.find(t.name);
    if (it == byname.end()) { set_err("tensor '%s': not a tensor of this configuration", t.name); return QDEC_REFUSED; }
    if (got.count(t.name)) { set_err("tensor '%s': given twice", t.name); return QDEC_REFUSED; }
    const Expect& e = *it->second;
    if (!known_type(t.type)) {
      set_err("tensor '%s': type %d unsupported (F32 = 0, Q4_0 = 2, Q8_0 = 8, Q4_K = 12, Q6_K = 14)", t.name, t.type);
      return QDEC_REFUSED;
    }
    if (is_kquant(t.type) && t.cols % 256) {
      set_err("tensor '%s': K-quant rows need a multiple of 256 values, got %lld", t.name, (long long)t.cols);
      return QDEC_REFUSED;
    }
    if (!e.matrix && t.type != kF32) { set_err("tensor '%s': norm gains and biases must be F32", t.name); return QDEC_REFUSED; }
    if (t.rows != e.rows || t.cols != e.cols) {
      set_err("tensor '%s': dims [%lld][%lld], expected [%lld][%lld]", t.name, (long long)t.rows, (long long)t.cols,
              (long long)e.rows, (long long)e.cols);
      return QDEC_REFUSED;
    }
    if (t.n_bytes != tensor_bytes(t.type, t.rows, t.cols)) {
      set_err("tensor '%s': %lld bytes, expected %lld", t.name, (long long)t.n_bytes,
              (long long)tensor_bytes(t.type, t.rows, t.cols));
      return QDEC_REFUSED;
    }
    if (!t.host_data) { set_err("tensor '%s': NULL data", t.name); return QDEC_REFUSED; }
    if (!scales_finite(t)) { set_err("tensor '%s': a block scale is not finite", t.name); return QDEC_REFUSED; }
    got[t.name] = &t;
  }
  for (auto& e : exp)
    if (e.required && !got.count(e.name)) { set_err("tensor '%s' is missing", e.name.c_str()); return QDEC_REFUSED; }
  for (int i = 0; i < c.n_layer; ++i) {
    std::string p = "blk." + std::to_string(i) + ".";
    if (got[p + "ffn_gate.weight"]->type != got[p + "ffn_up.weight"]->type) {
      set_err("layer %d: ffn_gate and ffn_up must share one type", i);
      return QDEC_REFUSED;
    }
  }

  qdec_model* m = new qdec_model();
  try {
    m->cfg = c;
    m->max_seqs = max_seqs;
    m->max_ctx = max_ctx;
    m->qd = c.n_head * c.head_dim;
    m->kd = c.n_head_kv * c.head_dim;
    m->nqkv = m->qd + 2 * m->kd;
    m->Fp = (int)(nblocks(c.ffn) * 32);
    const int H = c.hidden;
    auto TN = [&](const std::string& s) -> const qdec_tensor& { return *got.at(s); };

    {  // embedding / LM head
      const qdec_tensor& e = TN("token_embd.weight");
      Stage s(e.type, e.rows, nblocks(e.cols));
      for (int64_t r = 0; r < e.rows; ++r) s.put_row(r, e, r);
      m->embd = upload(m, s, (int)e.rows, (int)e.cols, (double)e.n_bytes, st);
      m->names[e.name] = NameRef{&m->embd, 0, (int)e.rows, (int)e.cols, 0, nullptr};
      m->tied = !got.count("output.weight");
      if (!m->tied) {
        const qdec_tensor& o = TN("output.weight");
        Stage so(o.type, o.rows, nblocks(o.cols));
        for (int64_t r = 0; r < o.rows; ++r) so.put_row(r, o, r);
        m->out_w = upload(m, so, (int)o.rows, (int)o.cols, (double)o.n_bytes, st);
        m->names[o.name] = NameRef{&m->out_w, 0, (int)o.rows, (int)o.cols, 0, nullptr};
      }
      m->output_norm = upload_vec(m, TN("output_norm.weight"), st);
    }
    m->layers.resize(c.n_layer);
    for (int i = 0; i < c.n_layer; ++i) {
      Layer& L = m->layers[i];
      std::string p = "blk." + std::to_string(i) + ".";
      L.global = c.window <= 0 || (i % c.window_period == c.window_period - 1);
      L.attn_norm = upload_vec(m, TN(p + "attn_norm.weight"), st);
      L.ffn_norm = upload_vec(m, TN(p + "ffn_norm.weight"), st);
      if (c.qk_norm) {
        L.q_norm = upload_vec(m, TN(p + "attn_q_norm.weight"), st);
        L.k_norm = upload_vec(m, TN(p + "attn_k_norm.weight"), st);
      }
      if (c.qkv_bias) {  // one fused q|k|v vector, in the row order of the fused matrix
        L.qkv_bias = m->dalloc<float>((size_t)m->nqkv);
        const char* part[3] = {"attn_q.bias", "attn_k.bias", "attn_v.bias"};
        const int off[3] = {0, m->qd, m->qd + m->kd};
        for (int j = 0; j < 3; ++j) {
          const qdec_tensor& tb = TN(p + part[j]);
          hipck(hipMemcpyAsync(L.qkv_bias + off[j], tb.host_data, (size_t)tb.cols * 4, hipMemcpyHostToDevice, st),
                "upload");
        }
      }
      if (c.sandwich_norm) {
        L.post_attn = upload_vec(m, TN(p + "post_attention_norm.weight"), st);
        L.post_ffw = upload_vec(m, TN(p + "post_ffw_norm.weight"), st);
      }
      const qdec_tensor &tq = TN(p + "attn_q.weight"), &tk = TN(p + "attn_k.weight"), &tv = TN(p + "attn_v.weight");
      L.qkv_split = tk.type != tq.type || tv.type != tq.type;
      if (L.qkv_split) {  // mixed types (K-quant files): one matrix each
        const qdec_tensor* part[3] = {&tq, &tk, &tv};
        for (int j = 0; j < 3; ++j) {
          const qdec_tensor& tj = *part[j];
          Stage s(tj.type, tj.rows, nblocks(H));
          for (int64_t r = 0; r < tj.rows; ++r) s.put_row(r, tj, r);
          L.qkv_part[j] = upload(m, s, (int)tj.rows, H, (double)tj.n_bytes, st);
          m->names[tj.name] = NameRef{&L.qkv_part[j], 0, (int)tj.rows, H, 0, nullptr};
        }
      } else {  // fused q|k|v rows
        Stage s(tq.type, m->nqkv, nblocks(H));
        for (int64_t r = 0; r < tq.rows; ++r) s.put_row(r, tq, r);
        for (int64_t r = 0; r < tk.rows; ++r) s.put_row(m->qd + r, tk, r);
        for (int64_t r = 0; r < tv.rows; ++r) s.put_row(m->qd + m->kd + r, tv, r);
        L.qkv = upload(m, s, m->nqkv, H, (double)(tq.n_bytes + tk.n_bytes + tv.n_bytes), st);
        m->names[tq.name] = NameRef{&L.qkv, 0, m->qd, H, 0, nullptr};
        m->names[tk.name] = NameRef{&L.qkv, m->qd, m->kd, H, 0, nullptr};
        m->names[tv.name] = NameRef{&L.qkv, m->qd + m->kd, m->kd, H, 0, nullptr};
      }
      {
        const qdec_tensor& to = TN(p + "attn_output.weight");
        Stage s(to.type, to.rows, nblocks(to.cols));
        for (int64_t r = 0; r < to.rows; ++r) s.put_row(r, to, r);
        L.o = upload(m, s, (int)to.rows, (int)to.cols, (double)to.n_bytes, st);
        m->names[to.name] = NameRef{&L.o, 0, (int)to.rows, (int)to.cols, 0, nullptr};
      }
      {  // gate/up interleaved in 32-row groups, zero rows up to Fp
        const qdec_tensor &tg = TN(p + "ffn_gate.weight"), &tu = TN(p + "ffn_up.weight");
        Stage s(tg.type, 2 * (int64_t)m->Fp, nblocks(H));
        for (int64_t r = 0; r < tg.rows; ++r) {
          int64_t gr = (r / 32) * 64 + (r % 32);
          s.put_row(gr, tg, r);
          s.put_row(gr + 32, tu, r);
        }
        L.gu = upload(m, s, 2 * m->Fp, H, (double)(tg.n_bytes + tu.n_bytes), st);
        m->names[tg.name] = NameRef{&L.gu, 0, c.ffn, H, 1, nullptr};
        m->names[tu.name] = NameRef{&L.gu, 0, c.ffn, H, 2, nullptr};
      }
      {
        const qdec_tensor& td = TN(p + "ffn_down.weight");
        Stage s(td.type, td.rows, nblocks(td.cols));
        for (int64_t r = 0; r < td.rows; ++r) s.put_row(r, td, r);
        L.down = upload(m, s, (int)td.rows, (int)td.cols, (double)td.n_bytes, st);
        m->names[td.name] = NameRef{&L.down, 0, (int)td.rows, (int)td.cols, 0, nullptr};
      }
    }
    {  // RoPE tables.  inv_freq[i] = 1 / theta^(i / half) in double, rounded once
       // to f32; angle = f32(pos) * inv_freq[i] as one f32 product; cos and sin
       // of that f32 angle in double, rounded once to f32.
      const int half = c.head_dim / 2;
      auto table = [&](double theta) {
        std::vector<float> inv(half);
        for (int i = 0; i < half; ++i) inv[i] = (float)(1.0 / std::pow(theta, (double)i / half));
        std::vector<float> t((size_t)max_ctx * half * 2);
        for (int p = 0; p < max_ctx; ++p)
          for (int i = 0; i < half; ++i) {
            const volatile float ang = (float)p * inv[i];
            t[((size_t)p * half + i) * 2] = (float)std::cos((double)ang);
            t[((size_t)p * half + i) * 2 + 1] = (float)std::sin((double)ang);
          }
        float2* d = m->dalloc<float2>((size_t)max_ctx * half);
        hipck(hipMemcpy(d, t.data(), t.size() * 4, hipMemcpyHostToDevice), "upload");
        return d;
      };
      m->rope_g = table(c.rope_theta);
      m->rope_l = c.window > 0 && c.rope_theta_local != c.rope_theta ? table(c.rope_theta_local) : m->rope_g;
      m->rope_cur = m->dalloc<float2>((size_t)2 * max_seqs * half);
    }
    // workspace rows (one prefill pass; the rings are sized by it)
    m->ws_T = std::max(std::min(max_ctx, 4096), max_seqs);
    // KV cache f32, per layer [B][nkv][positions][hd]
    layout_contiguous(m, st);
    // workspace
    const size_t T = m->ws_T;
    m->x = m->dalloc<float>(T * H);
    m->x2 = m->dalloc<float>(T * H);
    m->h = m->dalloc<float>(T * H);
    m->y = m->dalloc<float>(T * H);
    m->qkv = m->dalloc<float>(T * m->nqkv);
    m->q = m->dalloc<float>(T * m->qd);
    m->a = m->dalloc<float>(T * m->qd);
    m->m = m->dalloc<float>(T * m->Fp);
    hipck(hipMemsetAsync(m->m, 0, T * m->Fp * 4, st), "memset");
    {  // decode split over positions: at least four positions per lane group
       // (the first two pairs are requested at once); at max length about 8192
       // workgroups or more (several rounds of resident workgroups, so the last
       // round's partial fill costs little); at most kMaxChunks per (sequence,
       // KV head).  Past that bound the chunk grows by two positions per lane
       // group rather than doubling (chunks need not be a power of two in the
       // contiguous cache: 48 positions instead of 64 at head_dim 256 and 2,177
       // positions); a paged cache takes the next power of two, which divides
       // its pages.
      const double want = (double)max_ctx * c.n_head_kv * max_seqs / 8192.0;
      const int ng = 256 / (c.head_dim / 8);  // lane groups per workgroup
      int ch = 4 * ng;
      while (ch < want && ch < (1 << 30)) ch *= 2;
      const int64_t need = ((int64_t)max_ctx + kMaxChunks - 1) / kMaxChunks;
      if (ch < need) ch = (int)((need + 2 * ng - 1) / (2 * ng) * (2 * ng));
      int p2 = 1;
      while (p2 < ch) p2 *= 2;
      m->chunk = ch;
      m->chunk_base = p2;
      m->nchunk = (max_ctx + ch - 1) / ch;
    }
    m->acc_blk = (size_t)max_seqs * c.n_head * (c.head_dim + 1);
    m->acc = m->dalloc<float>(2 * kAccCopies * m->acc_blk);
    hipck(hipMemsetAsync(m->acc, 0, 2 * kAccCopies * m->acc_blk * sizeof(float), st), "memset");
    m->nvchunk = (c.vocab + kSampleChunk - 1) / kSampleChunk;
    m->s_v = m->dalloc<float>((size_t)max_seqs * m->nvchunk);
    m->s_i = m->dalloc<int>((size_t)max_seqs * m->nvchunk);
    // the LM head's waves: at most 1,024 workgroups of eight, or more when a
    // wave would otherwise hold more than 64 outputs (gemv's grid_min)
    m->am_n = std::max(8192, c.vocab / 64 + 64);
    m->am_v = m->dalloc<float>(m->am_n);
    m->am_i = m->dalloc<int>(m->am_n);
    m->cut_key = m->dalloc<uint32_t>(max_seqs);
    m->cut_idx = m->dalloc<int>(max_seqs);
    m->topp = TopPScratch{m->dalloc<float>((size_t)max_seqs * kTopPChunks), m->dalloc<int>((size_t)max_seqs * kTopPChunks),
                          m->dalloc<unsigned long long>((size_t)3 * max_seqs * 256),
                          m->dalloc<TopPState>((size_t)2 * max_seqs)};
    m->d_pos = m->dalloc<int>(64);
    m->d_tok = m->dalloc<int>(64);
    m->d_seq = m->dalloc<int>(64);
    m->seq_pages.assign(max_seqs, {});
    m->d_params = m->dalloc<StepParams>(1);
    hipck(hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking), "hipStreamCreate");
    m->d_prompt = m->dalloc<int>(T);
    hipck(hipHostMalloc((void**)&m->err_host, sizeof(int), hipHostMallocMapped), "hipHostMalloc");
    *m->err_host = 0;
    hipck(hipHostGetDevicePointer((void**)&m->err_dev, m->err_host, 0), "hipHostGetDevicePointer");
    m->kvlen.assign(max_seqs, 0);
    hipck(hipStreamSynchronize(st), "load sync");
  } catch (const HipError& e) {
    set_err("internal: %s", e.msg.c_str());
    drain(st);
    free_model(m);
    return QDEC_INTERNAL;
  } catch (const std::bad_alloc&) {
    set_err("host out of memory while loading");
    free_model(m);
    return QDEC_INTERNAL;
  }
  *out = m;
  return QDEC_OK;
}

// ------------------------------------------------------------ paged KV cache
// Pages are handed out from a free stack as sequences grow and returned on
// reset / truncate.  New page-table entries reach the device in stream order,
// as kernel arguments (table_set_kernel, or step_begin_kernel for decode), so
// no host buffer is read asynchronously.  A page returned by one call and
// handed to another sequence by a later call is safe because both calls' work
// runs in stream order on the caller's stream.
struct PageSet {
  std::vector<std::pair<int, int>> sets;  // (table index, page)
  std::vector<std::pair<int, int>> taken; // (seq, count) to roll back
};

// Make sequence seq hold pages for positions [0, len); false (nothing changed)
// when the free pages do not suffice.
bool grow_pages(qdec_model* m, int seq, int len, PageSet& ps) {
  if (!m->page_size) return true;
  const int need = (len + m->page_size - 1) >> m->log2p;
  auto& held = m->seq_pages[seq];
  const int add = need - (int)held.size();
  if (add <= 0) return true;
  if (add > (int)m->free_pages.size()) return false;
  for (int i = 0; i < add; ++i) {
    const int pg = m->free_pages.back();
    m->free_pages.pop_back();
    ps.sets.push_back({seq * m->table_w + (int)held.size(), pg});
    held.push_back(pg);
  }
  ps.taken.push_back({seq, add});
  return true;
}

void undo_pages(qdec_model* m, PageSet& ps) {
  for (auto it = ps.taken.rbegin(); it != ps.taken.rend(); ++it)
    for (int i = 0; i < it->second; ++i) {
      m->free_pages.push_back(m->seq_pages[it->first].back());
      m->seq_pages[it->first].pop_back();
    }
  ps.sets.clear();
  ps.taken.clear();
}

// Return the pages of seq past the first ceil(len / P).
void shrink_pages(qdec_model* m, int seq, int len) {
  if (!m->page_size) return;
  const int keep = (len + m->page_size - 1) >> m->log2p;
  auto& held = m->seq_pages[seq];
  while ((int)held.size() > keep) {
    m->free_pages.push_back(held.back());
    held.pop_back();
  }
}

void launch_table_sets(qdec_model* m, hipStream_t st, const PageSet& ps) {
  for (size_t i0 = 0; i0 < ps.sets.size(); i0 += 64) {
    TableSet t{};
    t.n = (int)std::min<size_t>(64, ps.sets.size() - i0);
    for (int i = 0; i < t.n; ++i) {
      t.idx[i] = ps.sets[i0 + i].first;
      t.val[i] = ps.sets[i0 + i].second;
    }
    t.table = m->d_table;
    Timed tm(m, st, "table_set", 0, 0);
    qlaunch(table_set_kernel, 1, 64, 0, st, t);
  }
}

// One decode step for rows 0..n-1.  seqs: the sequence slot of each row
// (host array, distinct), or null for rows = sequences 0..n-1.
int decode_impl(qdec_model* m, const int32_t* seqs, const int32_t* tokens, int32_t n_seqs, float* d_logits,
                int32_t* d_token_out, float temperature, float top_p, uint64_t seed, uint64_t step, uint32_t flags,
                hipStream_t st) {
  const qdec_config& c = m->cfg;
  if (n_seqs < 1 || n_seqs > m->max_seqs) { set_err("n_seqs %d outside [1, %d]", n_seqs, m->max_seqs); return QDEC_REFUSED; }
  if (!tokens || !d_logits || !d_token_out) { set_err("tokens, d_logits and d_token_out must not be NULL"); return QDEC_REFUSED; }
  if (!(temperature >= 0.f) || !std::isfinite(temperature)) { set_err("temperature must be finite and >= 0"); return QDEC_REFUSED; }
  if (std::isnan(top_p)) { set_err("top_p must not be NaN"); return QDEC_REFUSED; }
  if (flags & ~(uint32_t)QDEC_TOKENS_ON_DEVICE) { set_err("decode: unknown flag bits 0x%x", flags); return QDEC_REFUSED; }
  const bool on_dev = flags & QDEC_TOKENS_ON_DEVICE;
  std::vector<int> slot(n_seqs);
  std::vector<char> used(m->max_seqs, 0);
  for (int r = 0; r < n_seqs; ++r) {
    const int s = seqs ? seqs[r] : r;
    if (s < 0 || s >= m->max_seqs) { set_err("seqs[%d] = %d outside [0, %d)", r, s, m->max_seqs); return QDEC_REFUSED; }
    if (used[s]) { set_err("sequence %d appears twice in one step", s); return QDEC_REFUSED; }
    used[s] = 1;
    slot[r] = s;
    if (m->kvlen[s] >= m->max_ctx) { set_err("seq %d: KV cache full (max_ctx %d)", s, m->max_ctx); return QDEC_REFUSED; }
    if (!on_dev && (tokens[r] < 0 || tokens[r] >= c.vocab)) {
      set_err("tokens[%d] = %d outside [0, %d)", r, tokens[r], c.vocab);
      return QDEC_REFUSED;
    }
  }
  PageSet ps;
  for (int r = 0; r < n_seqs; ++r)
    if (!grow_pages(m, slot[r], m->kvlen[slot[r]] + 1, ps)) {
      undo_pages(m, ps);
      set_err("KV pages exhausted (%d pages of %d positions)", m->n_pages, m->page_size);
      return QDEC_REFUSED;
    }
  const bool slotted = seqs != nullptr;
  try {
    m->last_stream = st;
    m->row_seq = slot;
    StepArgs sa{};
    sa.n = n_seqs;
    for (int r = 0; r < n_seqs; ++r) {
      sa.pos[r] = m->kvlen[slot[r]];
      sa.host_tok[r] = on_dev ? 0 : tokens[r];
      sa.seq[r] = slot[r];
    }
    sa.d_seq = slotted ? m->d_seq : nullptr;
    sa.tbl_n = (int)ps.sets.size();  // at most one new page per row
    for (int i = 0; i < sa.tbl_n; ++i) {
      sa.tbl_idx[i] = ps.sets[i].first;
      sa.tbl_val[i] = ps.sets[i].second;
    }
    sa.d_table = m->d_table;
    sa.dev_tok = on_dev ? tokens : nullptr;
    sa.vocab = c.vocab;
    sa.d_pos = m->d_pos;
    sa.d_tok = m->d_tok;
    sa.err = m->err_dev;
    sa.params = StepParams{temperature, top_p, n_seqs, seed, step, d_logits, d_token_out};
    const bool topp = temperature > 0.f && top_p < 1.f;
    const bool greedy1 = n_seqs == 1 && !(temperature > 0.f);
    sa.d_params = m->d_params;
    sa.rope_g = m->rope_g;
    sa.rope_l = m->rope_l;
    sa.rope_cur = m->rope_cur;
    sa.half = c.head_dim / 2;
    sa.max_seqs = m->max_seqs;
    // attention of layer l clears the accumulators of layer l + 1's parity;
    // with an odd layer count the last layer has layer 0's parity, so the step
    // clears it here
    sa.acc_clear = c.n_layer % 2 ? m->acc : nullptr;
    sa.acc_n = (long)(kAccCopies * m->acc_blk);
    {
      Timed tm(m, st, "step_begin", 0, 0);
      qlaunch(step_begin_kernel, 1, 256, 0, st, sa);
    }
    if (m->timing) {
      decode_body(m, st, n_seqs, topp, slotted, greedy1);
    } else {
      // graph per (batch size, slotted, top-p on, fused greedy choice)
      hipGraphExec_t& ge = m->graphs[8 * n_seqs + (greedy1 ? 4 : 0) + (slotted ? 2 : 0) + (topp ? 1 : 0)];
      if (!ge) {
        hipGraph_t graph = nullptr;
        hipck(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture");
        try {
          decode_body(m, m->cap_stream, n_seqs, topp, slotted, greedy1);
        } catch (...) {
          (void)hipStreamEndCapture(m->cap_stream, &graph);
          if (graph) (void)hipGraphDestroy(graph);
          throw;
        }
        hipck(hipStreamEndCapture(m->cap_stream, &graph), "hipStreamEndCapture");
        hipError_t e = hipGraphInstantiate(&ge, graph, nullptr, nullptr, 0);
        (void)hipGraphDestroy(graph);
        hipck(e, "hipGraphInstantiate");
      }
      hipck(hipGraphLaunch(ge, st), "hipGraphLaunch");
    }
    for (int r = 0; r < n_seqs; ++r) m->kvlen[slot[r]] += 1;
  } catch (const HipError& e) {
    return fail_internal(m, st, e.msg);
  }
  return QDEC_OK;
}

}  // namespace

// ------------------------------------------------------------ allocation-free sampling
// qdec_sample_noalloc keeps its partial results in this file-scope device
// array instead of memory it allocates: per row, one (value, index) pair per
// 4,096-entry vocab chunk, and the top-p cut (key, index).  Offsets are fixed:
// values at 0, indices at 64 KiB, cut keys at 128 KiB, cut indices 256 bytes
// later.  Each GPU the library runs on holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device.
constexpr int kNoAllocRows = 64;
constexpr int kNoAllocVocab = 1 << 20;
constexpr size_t kNoAllocPart = (size_t)kNoAllocRows * (kNoAllocVocab / kSampleChunk) * 4;  // 64 KiB
// then the top-p passes': histograms [3][rows][256] u64, state [2][rows],
// chunk maxima and flags [rows][kTopPChunks]
constexpr size_t kNoAllocHist = 2 * kNoAllocPart + 2 * kNoAllocRows * 4;
constexpr size_t kNoAllocState = kNoAllocHist + (size_t)3 * kNoAllocRows * 256 * 8;
constexpr size_t kNoAllocPmax = kNoAllocState + (size_t)2 * kNoAllocRows * sizeof(TopPState);
constexpr size_t kNoAllocScratch = kNoAllocPmax + (size_t)2 * kNoAllocRows * kTopPChunks * 4;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratch];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of `scratch` on each device, once looked up

// The device address of `scratch` on the current device (looked up on the
// first call made on that device).  Null with the error text set on failure.
unsigned char* scratch_address() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_err("internal: hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= 64) {
    set_err("internal: device %d outside the 64 the scratch table holds", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      set_err("internal: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return static_cast<unsigned char*>(g_scratch_ptr[dev]);
}
}  // namespace

// ================================================================= C ABI
// Error text for the host-only sources of the library (model files).
__attribute__((visibility("hidden"))) void qdec_set_error_text(const std::string& s) { g_err = s; }

extern "C" {

int32_t qdec_abi_version(void) { return QDEC_ABI_VERSION; }

const char* qdec_last_error(void) { return g_err.c_str(); }

int qdec_load_weights(const qdec_config* cfg, const qdec_tensor* tensors, int32_t n_tensors, int32_t max_seqs,
                      int32_t max_ctx, void* stream, qdec_model** out) {
  g_err.clear();
  try {
    return load(cfg, tensors, n_tensors, max_seqs, max_ctx, (hipStream_t)stream, out);
  } catch (...) {
    set_err("internal: unexpected exception while loading");
    return QDEC_INTERNAL;
  }
}

int qdec_prefill(qdec_model* m, int32_t seq, const int32_t* tokens, int32_t n_tokens, float* d_logits,
                 int32_t* d_token_out, uint32_t flags, void* stream) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  hipStream_t st = (hipStream_t)stream;
  const qdec_config& c = m->cfg;
  if (seq < 0 || seq >= m->max_seqs) { set_err("seq %d outside [0, %d)", seq, m->max_seqs); return QDEC_REFUSED; }
  if (n_tokens <= 0) { set_err("n_tokens must be > 0"); return QDEC_REFUSED; }
  if (!tokens || !d_logits) { set_err("tokens and d_logits must not be NULL"); return QDEC_REFUSED; }
  if (flags & ~(uint32_t)QDEC_ALL_LOGITS) { set_err("prefill: unknown flag bits 0x%x", flags); return QDEC_REFUSED; }
  if ((int64_t)m->kvlen[seq] + n_tokens > m->max_ctx) {
    set_err("seq %d: kv_len %d + %d tokens exceeds max_ctx %d", seq, m->kvlen[seq], n_tokens, m->max_ctx);
    return QDEC_REFUSED;
  }
  for (int i = 0; i < n_tokens; ++i)
    if (tokens[i] < 0 || tokens[i] >= c.vocab) {
      set_err("tokens[%d] = %d outside [0, %d)", i, tokens[i], c.vocab);
      return QDEC_REFUSED;
    }
  const bool all = flags & QDEC_ALL_LOGITS;
  PageSet ps;
  if (!grow_pages(m, seq, m->kvlen[seq] + n_tokens, ps)) {
    set_err("KV pages exhausted (%d pages of %d positions)", m->n_pages, m->page_size);
    return QDEC_REFUSED;
  }
  try {
    m->last_stream = st;
    launch_table_sets(m, st, ps);
    const int H = c.hidden, V = c.vocab;
    const int pos_start = m->kvlen[seq];
    for (int c0 = 0; c0 < n_tokens; c0 += m->ws_T) {
      const int T = std::min(m->ws_T, n_tokens - c0);
      const int pos0 = pos_start + c0;
      const bool last = c0 + T == n_tokens;
      hipck(hipMemcpyAsync(m->d_prompt, tokens + c0, (size_t)T * 4, hipMemcpyHostToDevice, st), "token upload");
      embed(m, st, m->d_prompt, T, m->x);
      blocks(m, st, T, seq, pos0, nullptr);
      if (all) {
        rmsnorm_rows(m, st, m->x, H, m->output_norm, H, m->h, H, T, 0);
        gemm(m, st, m->lm(), m->h, H, T, d_logits + (size_t)c0 * V, V, kModeStore);
      } else if (last) {
        const int nw = gemv(m, st, m->lm(), m->x + (size_t)(T - 1) * H, H, m->output_norm, c.rms_eps, d_logits, V,
                            1, kModeStore, nullptr, Resid{}, nullptr, AccIn{}, d_token_out != nullptr);
        if (d_token_out) argmax_final(m, st, nw, d_token_out);
      }
      if (last && d_token_out && all) {
        const float* row = all ? d_logits + (size_t)(n_tokens - 1) * V : d_logits;
        sample(m, st, row, V, 1, 0.f, 0, 0, d_token_out, nullptr);
      }
    }
    m->kvlen[seq] += n_tokens;
  } catch (const HipError& e) {
    return fail_internal(m, st, e.msg);
  }
  return QDEC_OK;
}

int qdec_decode_step(qdec_model* m, const int32_t* tokens, int32_t n_seqs, float* d_logits, int32_t* d_token_out,
                     float temperature, float top_p, uint64_t seed, uint64_t step, uint32_t flags, void* stream) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  return decode_impl(m, nullptr, tokens, n_seqs, d_logits, d_token_out, temperature, top_p, seed, step, flags,
                     (hipStream_t)stream);
}

int qdec_decode_batch(qdec_model* m, const int32_t* seqs, const int32_t* tokens, int32_t n, float* d_logits,
                      int32_t* d_token_out, float temperature, float top_p, uint64_t seed, uint64_t step,
                      uint32_t flags, void* stream) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  if (!seqs) { set_err("seqs must not be NULL"); return QDEC_REFUSED; }
  return decode_impl(m, seqs, tokens, n, d_logits, d_token_out, temperature, top_p, seed, step, flags,
                     (hipStream_t)stream);
}

int qdec_kv_reset(qdec_model* m, int32_t seq) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  if (seq < -1 || seq >= m->max_seqs) { set_err("seq %d outside [-1, %d)", seq, m->max_seqs); return QDEC_REFUSED; }
  for (int s = 0; s < m->max_seqs; ++s)
    if (seq < 0 || s == seq) {
      m->kvlen[s] = 0;
      shrink_pages(m, s, 0);
    }
  return QDEC_OK;
}

int qdec_kv_truncate(qdec_model* m, int32_t seq, int32_t n) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  if (seq < 0 || seq >= m->max_seqs) { set_err("seq %d outside [0, %d)", seq, m->max_seqs); return QDEC_REFUSED; }
  if (n < 0 || n > m->kvlen[seq]) { set_err("n %d outside [0, kv_len %d]", n, m->kvlen[seq]); return QDEC_REFUSED; }
  // a ring has overwritten the slots of positions more than R - window behind
  // the length: the window of position n is still whole only this close
  for (int l = 0; l < m->cfg.n_layer; ++l)
    if (m->kv_ring[l] && m->kvlen[seq] - n > (1 << m->kv_ring[l]) - layer_window(m, l)) {
      set_err("seq %d: truncating %d positions exceeds the window layers' ring of %d positions (window %d); "
              "turn the ring off (qdec_kv_ring) to truncate further", seq, m->kvlen[seq] - n, 1 << m->kv_ring[l],
              layer_window(m, l));
      return QDEC_REFUSED;
    }
  m->kvlen[seq] = n;
  shrink_pages(m, seq, n);
  return QDEC_OK;
}

int qdec_kv_write(qdec_model* m, int32_t seq, int32_t layer, const float* d_k, const float* d_v, int32_t n_pos,
                  void* stream) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  hipStream_t st = (hipStream_t)stream;
  const qdec_config& c = m->cfg;
  if (seq < 0 || seq >= m->max_seqs) { set_err("seq %d outside [0, %d)", seq, m->max_seqs); return QDEC_REFUSED; }
  if (layer < 0 || layer >= c.n_layer) { set_err("layer %d outside [0, %d)", layer, c.n_layer); return QDEC_REFUSED; }
  if (n_pos < 0 || n_pos > m->max_ctx) { set_err("n_pos %d outside [0, %d]", n_pos, m->max_ctx); return QDEC_REFUSED; }
  if (n_pos > 0 && (!d_k || !d_v)) { set_err("d_k and d_v must not be NULL"); return QDEC_REFUSED; }
  PageSet ps;
  if (!grow_pages(m, seq, n_pos, ps)) {
    set_err("KV pages exhausted (%d pages of %d positions)", m->n_pages, m->page_size);
    return QDEC_REFUSED;
  }
  try {
    m->last_stream = st;
    launch_table_sets(m, st, ps);
    shrink_pages(m, seq, n_pos);
    if (n_pos) {
      // a ring keeps the last 2^ring positions (earlier ones would share their slots)
      const int j0 = m->kv_ring[layer] ? std::max(0, n_pos - (1 << m->kv_ring[layer])) : 0;
      KvScatter a{d_k, d_v, m->lkc(layer), m->lvc(layer), n_pos, c.n_head_kv, m->max_ctx, c.head_dim, seq,
                  m->lmap(layer), j0};
      Timed tm(m, st, "kv_scatter", (double)(n_pos - j0) * c.n_head_kv * c.head_dim * 16, 0);
      qlaunch(kv_scatter_kernel, dim3(n_pos - j0, c.n_head_kv, 2), 64, 0, st, a);
    }
    m->kvlen[seq] = n_pos;
  } catch (const HipError& e) {
    return fail_internal(m, st, e.msg);
  }
  return QDEC_OK;
}

int qdec_kv_paged(qdec_model* m, int32_t page_size, int32_t n_pages, void* stream) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  hipStream_t st = (hipStream_t)stream;
  const qdec_config& c = m->cfg;
  if (page_size < 16 || page_size > (1 << 20) || (page_size & (page_size - 1))) {
    set_err("page_size %d must be a power of two in [16, 2^20]", page_size);
    return QDEC_REFUSED;
  }
  if (n_pages < 1) { set_err("n_pages must be >= 1"); return QDEC_REFUSED; }
  for (int s = 0; s < m->max_seqs; ++s)
    if (m->kvlen[s]) {
      set_err("the KV cache is in use (seq %d holds %d positions): reset it first", s, m->kvlen[s]);
      return QDEC_REFUSED;
    }
  // a decode chunk lies in one page: chunks of min(chunk, page_size) positions,
  // at least the kernel's minimum and at most kMaxChunks of them per sequence
  const int ch_min = 4 * (256 / (c.head_dim / 8));
  if (page_size < ch_min) {
    set_err("page_size %d is below the decode chunk of %d positions at head_dim %d", page_size, ch_min, c.head_dim);
    return QDEC_REFUSED;
  }
  const int chunk = std::min(m->chunk_base, page_size);
  const int nchunk = (m->max_ctx + chunk - 1) / chunk;
  if (nchunk > kMaxChunks) {
    int need = 1;
    while ((int64_t)need * kMaxChunks < m->max_ctx) need *= 2;
    set_err("page_size %d is too small for max_ctx %d (at least %d)", page_size, m->max_ctx, need);
    return QDEC_REFUSED;
  }
  if ((int64_t)n_pages * c.n_head_kv * page_size >= INT32_MAX) {
    set_err("a pool of %d pages of %d positions holds 2^31 cache rows per layer or more", n_pages, page_size);
    return QDEC_REFUSED;
  }
  const size_t layer = (size_t)n_pages * c.n_head_kv * page_size * c.head_dim;
  if ((double)layer * c.n_layer * 8.0 > 256.0 * (1ull << 30)) {
    set_err("a pool of %d pages of %d positions needs more than 256 GiB", n_pages, page_size);
    return QDEC_REFUSED;
  }
  try {
    m->last_stream = st;
    hipck(hipStreamSynchronize(st), "sync");  // nothing reads the old cache any more
    for (auto& g : m->graphs)  // captured with the old cache and kernels
      if (g.second) (void)hipGraphExecDestroy(g.second);
    m->graphs.clear();
    m->dfree(m->kc);
    m->dfree(m->vc);
    m->kc = m->vc = nullptr;
    if (m->d_table) m->dfree(m->d_table);
    m->kc = m->dalloc<float>(layer * c.n_layer);
    m->vc = m->dalloc<float>(layer * c.n_layer);
    hipck(hipMemsetAsync(m->kc, 0, layer * c.n_layer * 4, st), "memset");
    hipck(hipMemsetAsync(m->vc, 0, layer * c.n_layer * 4, st), "memset");
    m->table_w = (m->max_ctx + page_size - 1) / page_size;
    m->d_table = m->dalloc<int>((size_t)m->max_seqs * m->table_w);
    hipck(hipMemsetAsync(m->d_table, 0, (size_t)m->max_seqs * m->table_w * 4, st), "memset");
    m->chunk = chunk;
    m->nchunk = nchunk;
    m->kv_layer = layer;
    m->kv_off.assign(c.n_layer, 0);
    for (int l = 0; l < c.n_layer; ++l) m->kv_off[l] = (size_t)l * layer;
    m->kv_ring.assign(c.n_layer, 0);  // pages hold every position
    m->page_size = page_size;
    m->log2p = 0;
    while ((1 << m->log2p) < page_size) ++m->log2p;
    m->n_pages = n_pages;
    m->free_pages.resize(n_pages);
    for (int i = 0; i < n_pages; ++i) m->free_pages[i] = n_pages - 1 - i;  // page 0 handed out first
    m->seq_pages.assign(m->max_seqs, {});
    hipck(hipStreamSynchronize(st), "sync");
  } catch (const HipError& e) {
    return fail_internal(m, st, e.msg);
  }
  return QDEC_OK;
}

int qdec_kv_pages(const qdec_model* m, int32_t* page_size, int32_t* n_pages, int32_t* n_free) {
  g_err.clear();
  if (!m || !page_size || !n_pages || !n_free) { set_err("model and outputs must not be NULL"); return QDEC_REFUSED; }
  *page_size = m->page_size;
  *n_pages = m->n_pages;
  *n_free = (int32_t)m->free_pages.size();
  return QDEC_OK;
}

int qdec_kv_ring(qdec_model* m, int32_t enable, void* stream) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (enable != 0 && enable != 1) { set_err("enable must be 0 or 1"); return QDEC_REFUSED; }
  if (m->page_size) { set_err("the cache is paged: its pages hold every position"); return QDEC_REFUSED; }
  for (int s = 0; s < m->max_seqs; ++s)
    if (m->kvlen[s]) {
      set_err("the KV cache is in use (seq %d holds %d positions): reset it first", s, m->kvlen[s]);
      return QDEC_REFUSED;
    }
  if ((enable == 1) == m->ring_on) return QDEC_OK;
  try {
    m->last_stream = st;
    hipck(hipStreamSynchronize(st), "sync");  // nothing reads the old cache any more
    for (auto& g : m->graphs)  // captured with the old cache
      if (g.second) (void)hipGraphExecDestroy(g.second);
    m->graphs.clear();
    m->dfree(m->kc);
    m->dfree(m->vc);
    m->kc = m->vc = nullptr;
    m->ring_on = enable == 1;
    layout_contiguous(m, st);
    hipck(hipStreamSynchronize(st), "sync");
  } catch (const HipError& e) {
    return fail_internal(m, st, e.msg);
  }
  return QDEC_OK;
}

int qdec_kv_ring_positions(const qdec_model* m, int32_t layer, int32_t* out) {
  g_err.clear();
  if (!m || !out) { set_err("model and out must not be NULL"); return QDEC_REFUSED; }
  if (layer < 0 || layer >= m->cfg.n_layer) { set_err("layer %d outside [0, %d)", layer, m->cfg.n_layer); return QDEC_REFUSED; }
  *out = m->kv_ring[layer] ? 1 << m->kv_ring[layer] : 0;
  return QDEC_OK;
}

int qdec_kv_len(const qdec_model* m, int32_t seq, int32_t* out) {
  g_err.clear();
  if (!m || !out) { set_err("model and out must not be NULL"); return QDEC_REFUSED; }
  if (seq < 0 || seq >= m->max_seqs) { set_err("seq %d outside [0, %d)", seq, m->max_seqs); return QDEC_REFUSED; }
  *out = m->kvlen[seq];
  return QDEC_OK;
}

int qdec_poisoned(const qdec_model* m) { return m ? (m->poisoned ? 1 : 0) : -1; }

int qdec_decode_chunks(const qdec_model* m, int32_t* chunk, int32_t* n_chunks) {
  g_err.clear();
  if (!m || !chunk || !n_chunks) { set_err("model and outputs must not be NULL"); return QDEC_REFUSED; }
  *chunk = m->chunk;
  *n_chunks = m->nchunk;
  return QDEC_OK;
}

int qdec_debug_inject_fault(qdec_model* m, int32_t where) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  if (where != 0 && where != 1) { set_err("where must be 0 (disarm) or 1 (arm), got %d", where); return QDEC_REFUSED; }
  m->inject_fault = where;
  return QDEC_OK;
}

int qdec_set_prefill_precision(qdec_model* m, int32_t precision) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  if (precision != QDEC_PREFILL_F32 && precision != QDEC_PREFILL_BF16X3 && precision != QDEC_PREFILL_BF16) {
    set_err("unknown prefill precision %d", precision);
    return QDEC_REFUSED;
  }
  m->prefill_prec = precision;
  return QDEC_OK;
}

int qdec_free(qdec_model* m) {
  g_err.clear();
  if (!m) { set_err("model handle is NULL"); return QDEC_REFUSED; }
  drain(m->last_stream);
  (void)hipDeviceSynchronize();
  free_model(m);
  return QDEC_OK;
}

int qdec_debug_dequant(qdec_model* m, const char* name, float* d_out, void* stream) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  if (!name || !d_out) { set_err("name and d_out must not be NULL"); return QDEC_REFUSED; }
  auto it = m->names.find(name);
  if (it == m->names.end()) { set_err("no loaded matrix named '%s'", name); return QDEC_REFUSED; }
  const NameRef& r = it->second;
  hipStream_t st = (hipStream_t)stream;
  try {
    DequantArgs a{WView{r.mat->qs, r.mat->d, r.mat->type, r.mat->nblk, r.mat->sd}, nullptr, r.row_off, r.rows, r.cols, r.pair, d_out};
    Timed tm(m, st, "dequant", 0, 0);
    qlaunch(dequant_kernel, r.rows, 256, 0, st, a);
  } catch (const HipError& e) {
    return fail_internal(m, st, e.msg);
  }
  return QDEC_OK;
}

int qdec_debug_embed(qdec_model* m, const int32_t* d_tokens, int32_t n, float* d_out, void* stream) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  if (!d_tokens || !d_out || n <= 0) { set_err("d_tokens, d_out must not be NULL and n > 0"); return QDEC_REFUSED; }
  hipStream_t st = (hipStream_t)stream;
  try {
    embed(m, st, d_tokens, n, d_out);
  } catch (const HipError& e) {
    return fail_internal(m, st, e.msg);
  }
  return QDEC_OK;
}

int qdec_debug_sample(const float* d_logits, int32_t rows, int32_t vocab, float temperature, float top_p,
                      uint64_t seed, uint64_t step, int32_t* d_out, void* stream) {
  g_err.clear();
  if (!d_logits || !d_out || rows <= 0 || vocab <= 0) { set_err("bad arguments"); return QDEC_REFUSED; }
  if (!(temperature >= 0.f) || !std::isfinite(temperature)) { set_err("temperature must be finite and >= 0"); return QDEC_REFUSED; }
  if (std::isnan(top_p)) { set_err("top_p must not be NaN"); return QDEC_REFUSED; }
  hipStream_t st = (hipStream_t)stream;
  const int nch = (vocab + kSampleChunk - 1) / kSampleChunk;
  const bool topp = temperature > 0.f && top_p < 1.f;
  float* pv = nullptr;
  int* pi = nullptr;
  uint32_t* ck = nullptr;
  int* ci = nullptr;
  TopPScratch tp{};
  auto release = [&]() {
    (void)hipFree(pv);
    (void)hipFree(pi);
    (void)hipFree(ck);
    (void)hipFree(ci);
    (void)hipFree(tp.pmax);
    (void)hipFree(tp.pbad);
    (void)hipFree(tp.hist);
    (void)hipFree(tp.state);
  };
  if (hipMalloc(&pv, (size_t)rows * nch * 4) != hipSuccess || hipMalloc(&pi, (size_t)rows * nch * 4) != hipSuccess ||
      hipMalloc(&ck, (size_t)rows * 4) != hipSuccess || hipMalloc(&ci, (size_t)rows * 4) != hipSuccess ||
      hipMalloc(&tp.pmax, (size_t)rows * kTopPChunks * 4) != hipSuccess ||
      hipMalloc(&tp.pbad, (size_t)rows * kTopPChunks * 4) != hipSuccess ||
      hipMalloc(&tp.hist, (size_t)3 * rows * 256 * 8) != hipSuccess ||
      hipMalloc(&tp.state, (size_t)2 * rows * sizeof(TopPState)) != hipSuccess) {
    release();
    set_err("internal: hipMalloc failed");
    return QDEC_INTERNAL;
  }
  SampleArgs a{d_logits, vocab, vocab, rows, temperature, seed, step, pv, pi, nch, d_out, nullptr, nullptr,
               topp ? ck : nullptr, topp ? ci : nullptr};
  if (topp) topp_cut(st, TopPArgs{d_logits, vocab, vocab, rows, temperature, top_p, ck, ci, nullptr, tp.pmax, tp.pbad,
                                  tp.hist, tp.state, 0});
  qlaunch(sample_stage1_kernel, dim3(nch, rows), 256, 0, st, a);
  qlaunch(sample_stage2_kernel, rows, 64, 0, st, a);
  hipError_t e = hipStreamSynchronize(st);
  release();
  if (e != hipSuccess) { set_err("internal: %s", hipGetErrorString(e)); return QDEC_INTERNAL; }
  return QDEC_OK;
}

int qdec_sample_noalloc(const float* d_logits, int32_t rows, int32_t vocab, float temperature, float top_p,
                        uint64_t seed, uint64_t step, int32_t* d_out, void* stream) {
  g_err.clear();
  if (!d_logits || !d_out) { set_err("d_logits and d_out must not be NULL"); return QDEC_REFUSED; }
  if (rows < 1 || rows > kNoAllocRows) {
    set_err("rows %d outside [1, %d] (the fixed scratch holds %d rows)", rows, kNoAllocRows, kNoAllocRows);
    return QDEC_REFUSED;
  }
  if (vocab < 1 || vocab > kNoAllocVocab) {
    set_err("vocab %d outside [1, %d] (the fixed scratch holds %d chunks of %d per row)", vocab, kNoAllocVocab,
            kNoAllocVocab / kSampleChunk, kSampleChunk);
    return QDEC_REFUSED;
  }
  if (!(temperature >= 0.f) || !std::isfinite(temperature)) { set_err("temperature must be finite and >= 0"); return QDEC_REFUSED; }
  if (std::isnan(top_p)) { set_err("top_p must not be NaN"); return QDEC_REFUSED; }
  unsigned char* ptr = scratch_address();
  if (!ptr) return QDEC_INTERNAL;
  hipStream_t st = (hipStream_t)stream;
  const int nch = (vocab + kSampleChunk - 1) / kSampleChunk;
  const bool topp = temperature > 0.f && top_p < 1.f;
  float* pv = reinterpret_cast<float*>(ptr);
  int* pi = reinterpret_cast<int*>(ptr + kNoAllocPart);
  uint32_t* ck = reinterpret_cast<uint32_t*>(ptr + 2 * kNoAllocPart);
  int* ci = reinterpret_cast<int*>(ptr + 2 * kNoAllocPart + kNoAllocRows * 4);
  // every partial the sampling kernels read is written first in the same call
  // (stage 1 writes all rows x chunks, the top-p cut all rows): nothing to clear
  SampleArgs a{d_logits, vocab, vocab, rows, temperature, seed, step, pv, pi, nch, d_out, nullptr, nullptr,
               topp ? ck : nullptr, topp ? ci : nullptr};
  static_assert(kNoAllocHist % 8 == 0 && kNoAllocState % 8 == 0 && kNoAllocPmax % 8 == 0, "8-byte alignment");
  TopPArgs t{d_logits, vocab, vocab, rows, temperature, top_p, ck, ci, nullptr,
             reinterpret_cast<float*>(ptr + kNoAllocPmax),
             reinterpret_cast<int*>(ptr + kNoAllocPmax + (size_t)kNoAllocRows * kTopPChunks * 4),
             reinterpret_cast<unsigned long long*>(ptr + kNoAllocHist), reinterpret_cast<TopPState*>(ptr + kNoAllocState),
             0};
  try {
    if (topp) topp_cut(st, t);
    qlaunch(sample_stage1_kernel, dim3(nch, rows), 256, 0, st, a);
    qlaunch(sample_stage2_kernel, rows, 64, 0, st, a);
    hipck(hipGetLastError(), "sampling launch");
  } catch (const HipError& e) {
    set_err("internal: %s", e.msg.c_str());
    return QDEC_INTERNAL;
  }
  return QDEC_OK;
}

int qdec_debug_matmul(int32_t type, int64_t rows, int64_t cols, const void* host_data, int64_t n_bytes,
                      const float* d_x, int32_t n_x, float* d_y, int32_t precision, void* stream) {
  g_err.clear();
  if (precision != QDEC_PREFILL_F32 && precision != QDEC_PREFILL_BF16X3 && precision != QDEC_PREFILL_BF16) {
    set_err("unknown prefill precision %d", precision);
    return QDEC_REFUSED;
  }
  if (!known_type(type)) { set_err("type %d unsupported", type); return QDEC_REFUSED; }
  if (is_kquant(type) && cols % 256) { set_err("K-quant rows need a multiple of 256 values"); return QDEC_REFUSED; }
  if (rows <= 0 || cols <= 0 || rows > (1 << 24) || cols > (1 << 20) || !host_data || !d_x || !d_y || n_x <= 0) {
    set_err("bad arguments");
    return QDEC_REFUSED;
  }
  if (n_bytes != tensor_bytes(type, rows, cols)) { set_err("n_bytes %lld, expected %lld", (long long)n_bytes, (long long)tensor_bytes(type, rows, cols)); return QDEC_REFUSED; }
  hipStream_t st = (hipStream_t)stream;
  qdec_model tmp;  // holds the allocations only
  int rc = QDEC_OK;
  try {
    qdec_tensor t{"w", type, rows, cols, host_data, n_bytes};
    Stage s(type, rows, nblocks(cols));
    for (int64_t r = 0; r < rows; ++r) s.put_row(r, t, r);
    Mat w = upload(&tmp, s, (int)rows, (int)cols, (double)n_bytes, st);
    const int kp = w.nblk * 32;
    if (n_x <= 16) gemv(nullptr, st, w, d_x, kp, nullptr, 0.f, d_y, (int)rows, n_x, kModeStore);
    else gemm(nullptr, st, w, d_x, kp, n_x, d_y, (int)rows, kModeStore, precision);
    hipck(hipStreamSynchronize(st), "matmul sync");
  } catch (const HipError& e) {
    set_err("internal: %s", e.msg.c_str());
    rc = QDEC_INTERNAL;
  }
  for (void* p : tmp.allocs) (void)hipFree(p);
  tmp.allocs.clear();
  return rc;
}

int qdec_kernel_timing(qdec_model* m, int32_t enable, qdec_kstat* out, int32_t max_out, int32_t* n_out) {
  g_err.clear();
  if (int rc = check_usable(m)) return rc;
  if (enable) {
    try {
      while (m->evpool.size() < (1u << 17)) {
        hipEvent_t e;
        hipck(hipEventCreateWithFlags(&e, hipEventDisableSystemFence), "hipEventCreate");
        m->evpool.push_back(e);
      }
    } catch (const HipError& e) {
      return fail_internal(m, m->last_stream, e.msg);
    }
    m->evnext = 0;
    m->timing = true;
    return QDEC_OK;
  }
  m->timing = false;
  try {
    if (m->last_stream || !m->krecs.empty()) hipck(hipDeviceSynchronize(), "timing sync");
    std::vector<qdec_kstat> agg;
    for (auto& r : m->krecs) {
      float ms = 0.f;
      hipck(hipEventElapsedTime(&ms, r.a, r.b), "hipEventElapsedTime");
      auto it = std::find_if(agg.begin(), agg.end(), [&](const qdec_kstat& k) { return std::strcmp(k.name, r.cls) == 0; });
      if (it == agg.end()) {
        qdec_kstat k{};
        std::snprintf(k.name, sizeof(k.name), "%s", r.cls);
        agg.push_back(k);
        it = agg.end() - 1;
      }
      it->launches += 1;
      it->total_ms += ms;
      it->bytes += r.bytes;
      it->flops += r.flops;
    }
    m->krecs.clear();
    m->evnext = 0;
    int k = 0;
    for (; k < (int)agg.size() && k < max_out && out; ++k) out[k] = agg[k];
    if (n_out) *n_out = k;
  } catch (const HipError& e) {
    return fail_internal(m, m->last_stream, e.msg);
  }
  return QDEC_OK;
}

}  // extern "C"
