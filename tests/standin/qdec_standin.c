/*
 * A stand-in for libqdec.so with no GPU: every function declared in
 * include/qdec.h, recording each call, for host-only tests of the Python
 * binding (tessl `python/README.md`, "Build and test": the binding is tested
 * against a recording stand-in of its C library, and the library path is
 * overridden by an environment variable, here QDEC_LIB).
 *
 * Handles are heap records that are never released, so a second qdec_free of
 * the same handle is detected and counted instead of corrupting memory.  The
 * status of the next call can be forced (standin_force), and a forced status 2
 * latches the handle as poisoned, as the real library does.  No call does any
 * arithmetic of the forward pass.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/qdec.h"

#define MAGIC_LIVE 0x51444543u
#define MAGIC_FREED 0xdeadbeefu

struct qdec_model {
  unsigned magic;
  int poisoned;
  int max_seqs, max_ctx, vocab;
  int kvlen[64];
};

static char g_log[1 << 16];
static size_t g_log_len;
static char g_err[256];
static int g_force_status, g_frees, g_double_frees;

static void rec(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
#include <stdarg.h>
static void rec(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  int n = vsnprintf(g_log + g_log_len, sizeof(g_log) - g_log_len, fmt, ap);
  va_end(ap);
  if (n > 0 && g_log_len + (size_t)n + 1 < sizeof(g_log)) {
    g_log_len += (size_t)n;
    g_log[g_log_len++] = '\n';
    g_log[g_log_len] = 0;
  }
}

/* ---- control of the stand-in (not part of the ABI) ---- */
void standin_reset(void) {
  g_log_len = 0;
  g_log[0] = 0;
  g_force_status = 0;
  g_frees = g_double_frees = 0;
}
const char* standin_log(void) { return g_log; }
void standin_force(int status) { g_force_status = status; }
int standin_frees(void) { return g_frees; }
int standin_double_frees(void) { return g_double_frees; }

/* status of a call on handle m: a NULL / freed / poisoned handle is refused,
 * otherwise the forced status (once) or 0 */
static int status_of(qdec_model* m, const char* name) {
  if (!m) {
    snprintf(g_err, sizeof g_err, "%s: model handle is NULL", name);
    return QDEC_REFUSED;
  }
  if (m->magic != MAGIC_LIVE) {
    snprintf(g_err, sizeof g_err, "%s: handle already freed", name);
    return QDEC_REFUSED;
  }
  if (m->poisoned) {
    snprintf(g_err, sizeof g_err, "poisoned: free and load again");
    return QDEC_REFUSED;
  }
  int s = g_force_status;
  g_force_status = 0;
  if (s == QDEC_INTERNAL) {
    m->poisoned = 1;
    snprintf(g_err, sizeof g_err, "internal: forced by the stand-in");
  } else if (s == QDEC_REFUSED) {
    snprintf(g_err, sizeof g_err, "refused: forced by the stand-in");
  }
  return s;
}

int32_t qdec_abi_version(void) { return QDEC_ABI_VERSION; }
const char* qdec_last_error(void) { return g_err; }

int qdec_load_weights(const qdec_config* cfg, const qdec_tensor* t, int32_t n, int32_t max_seqs, int32_t max_ctx,
                      void* stream, qdec_model** out) {
  rec("load_weights n_tensors=%d max_seqs=%d max_ctx=%d stream=%p", n, max_seqs, max_ctx, stream);
  if (!cfg || !out || max_seqs < 1 || max_seqs > 64) {
    snprintf(g_err, sizeof g_err, "bad arguments");
    return QDEC_REFUSED;
  }
  for (int i = 0; i < n; ++i)
    if (!t[i].name || !t[i].host_data) {
      snprintf(g_err, sizeof g_err, "tensor %d: NULL name or data", i);
      return QDEC_REFUSED;
    }
  qdec_model* m = (qdec_model*)calloc(1, sizeof(qdec_model));
  m->magic = MAGIC_LIVE;
  m->max_seqs = max_seqs;
  m->max_ctx = max_ctx;
  m->vocab = cfg->vocab;
  *out = m;
  return QDEC_OK;
}

int qdec_gguf_config(const char* path, const char* archdef, qdec_config* out) {
  rec("gguf_config %s", path ? path : "(null)");
  (void)archdef;
  (void)out;
  snprintf(g_err, sizeof g_err, "stand-in: no files");
  return QDEC_REFUSED;
}
int qdec_load_gguf(const char* path, const char* archdef, int32_t max_seqs, int32_t max_ctx, void* stream,
                   qdec_model** out) {
  rec("load_gguf %s", path ? path : "(null)");
  (void)archdef; (void)max_seqs; (void)max_ctx; (void)stream; (void)out;
  snprintf(g_err, sizeof g_err, "stand-in: no files");
  return QDEC_REFUSED;
}
const char* qdec_archdef_builtin(const char* arch) { (void)arch; return NULL; }

int qdec_prefill(qdec_model* m, int32_t seq, const int32_t* tokens, int32_t n, float* d_logits, int32_t* d_tok,
                 uint32_t flags, void* stream) {
  rec("prefill seq=%d n=%d flags=%u", seq, n, flags);
  (void)tokens; (void)d_logits; (void)d_tok; (void)stream;
  int s = status_of(m, "prefill");
  if (s == 0 && seq >= 0 && seq < m->max_seqs) m->kvlen[seq] += n;
  return s;
}
int qdec_decode_step(qdec_model* m, const int32_t* tokens, int32_t n, float* d_logits, int32_t* d_tok, float temp,
                     float top_p, uint64_t seed, uint64_t step, uint32_t flags, void* stream) {
  rec("decode_step n=%d temp=%g top_p=%g seed=%llu step=%llu flags=%u", n, temp, top_p, (unsigned long long)seed,
      (unsigned long long)step, flags);
  (void)tokens; (void)d_logits; (void)d_tok; (void)stream;
  return status_of(m, "decode_step");
}
int qdec_decode_batch(qdec_model* m, const int32_t* seqs, const int32_t* tokens, int32_t n, float* d_logits,
                      int32_t* d_tok, float temp, float top_p, uint64_t seed, uint64_t step, uint32_t flags,
                      void* stream) {
  rec("decode_batch n=%d", n);
  (void)seqs; (void)tokens; (void)d_logits; (void)d_tok; (void)temp; (void)top_p; (void)seed; (void)step;
  (void)flags; (void)stream;
  return status_of(m, "decode_batch");
}
int qdec_kv_paged(qdec_model* m, int32_t page_size, int32_t n_pages, void* stream) {
  rec("kv_paged %d %d", page_size, n_pages);
  (void)stream;
  return status_of(m, "kv_paged");
}
int qdec_kv_ring(qdec_model* m, int32_t enable, void* stream) {
  rec("kv_ring %d", enable);
  (void)stream;
  return status_of(m, "kv_ring");
}
int qdec_kv_ring_positions(const qdec_model* m, int32_t layer, int32_t* out) {
  rec("kv_ring_positions %d", layer);
  if (!m || !out) return QDEC_REFUSED;
  *out = 0;
  return QDEC_OK;
}
int qdec_kv_pages(const qdec_model* m, int32_t* page_size, int32_t* n_pages, int32_t* n_free) {
  rec("kv_pages");
  if (!m || !page_size || !n_pages || !n_free) return QDEC_REFUSED;
  *page_size = *n_pages = *n_free = 0;
  return QDEC_OK;
}
int qdec_kv_reset(qdec_model* m, int32_t seq) {
  rec("kv_reset %d", seq);
  int s = status_of(m, "kv_reset");
  if (s == 0)
    for (int i = 0; i < m->max_seqs; ++i)
      if (seq < 0 || i == seq) m->kvlen[i] = 0;
  return s;
}
int qdec_kv_truncate(qdec_model* m, int32_t seq, int32_t n) {
  rec("kv_truncate %d %d", seq, n);
  int s = status_of(m, "kv_truncate");
  if (s == 0 && seq >= 0 && seq < m->max_seqs && n >= 0 && n <= m->kvlen[seq]) m->kvlen[seq] = n;
  return s;
}
int qdec_kv_write(qdec_model* m, int32_t seq, int32_t layer, const float* d_k, const float* d_v, int32_t n_pos,
                  void* stream) {
  rec("kv_write %d %d %d", seq, layer, n_pos);
  (void)d_k; (void)d_v; (void)stream;
  return status_of(m, "kv_write");
}
int qdec_kv_len(const qdec_model* m, int32_t seq, int32_t* out) {
  rec("kv_len %d", seq);
  if (!m || !out || seq < 0 || seq >= m->max_seqs) return QDEC_REFUSED;
  *out = m->kvlen[seq];
  return QDEC_OK;
}
int qdec_decode_chunks(const qdec_model* m, int32_t* chunk, int32_t* n_chunks) {
  rec("decode_chunks");
  if (!m || !chunk || !n_chunks) return QDEC_REFUSED;
  *chunk = 64;
  *n_chunks = 1;
  return QDEC_OK;
}
int qdec_set_prefill_precision(qdec_model* m, int32_t precision) {
  rec("set_prefill_precision %d", precision);
  return status_of(m, "set_prefill_precision");
}
int qdec_poisoned(const qdec_model* m) { return m ? (m->poisoned ? 1 : 0) : -1; }
int qdec_free(qdec_model* m) {
  rec("free");
  if (!m) return QDEC_REFUSED;
  if (m->magic != MAGIC_LIVE) {
    ++g_double_frees;
    return QDEC_REFUSED;
  }
  m->magic = MAGIC_FREED; /* kept allocated: a second free is detected */
  ++g_frees;
  return QDEC_OK;
}
int qdec_debug_dequant(qdec_model* m, const char* name, float* d_out, void* stream) {
  rec("debug_dequant %s", name ? name : "(null)");
  (void)d_out; (void)stream;
  return status_of(m, "debug_dequant");
}
int qdec_debug_embed(qdec_model* m, const int32_t* d_tokens, int32_t n, float* d_out, void* stream) {
  rec("debug_embed %d", n);
  (void)d_tokens; (void)d_out; (void)stream;
  return status_of(m, "debug_embed");
}
int qdec_debug_sample(const float* d_logits, int32_t rows, int32_t vocab, float temp, float top_p, uint64_t seed,
                      uint64_t step, int32_t* d_out, void* stream) {
  rec("debug_sample %d %d", rows, vocab);
  (void)d_logits; (void)temp; (void)top_p; (void)seed; (void)step; (void)d_out; (void)stream;
  return QDEC_REFUSED;
}
int qdec_sample_noalloc(const float* d_logits, int32_t rows, int32_t vocab, float temp, float top_p, uint64_t seed,
                        uint64_t step, int32_t* d_out, void* stream) {
  rec("sample_noalloc %d %d", rows, vocab);
  (void)d_logits; (void)temp; (void)top_p; (void)seed; (void)step; (void)d_out; (void)stream;
  return QDEC_REFUSED;
}
int qdec_debug_matmul(int32_t type, int64_t rows, int64_t cols, const void* host_data, int64_t n_bytes,
                      const float* d_x, int32_t n_x, float* d_y, int32_t precision, void* stream) {
  rec("debug_matmul %d", type);
  (void)rows; (void)cols; (void)host_data; (void)n_bytes; (void)d_x; (void)n_x; (void)d_y; (void)precision;
  (void)stream;
  return QDEC_REFUSED;
}
int qdec_debug_inject_fault(qdec_model* m, int32_t where) {
  rec("debug_inject_fault %d", where);
  int s = status_of(m, "debug_inject_fault");
  if (s == 0 && where == 1) g_force_status = QDEC_INTERNAL;
  return s;
}
int qdec_kernel_timing(qdec_model* m, int32_t enable, qdec_kstat* out, int32_t max_out, int32_t* n_out) {
  rec("kernel_timing %d", enable);
  (void)out; (void)max_out;
  if (n_out) *n_out = 0;
  return status_of(m, "kernel_timing");
}
