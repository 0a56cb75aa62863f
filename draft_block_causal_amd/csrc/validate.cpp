// Host-only argument validation and workspace layout of the Domino C ABI.
// Pure C++ (no HIP calls), so it can also be built and sanitised on a CPU.
#include "validate.h"
#include "kernels.h"

#include "psplit.h"

#include <cmath>
#include <initializer_list>

namespace domino {

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dtype) { return dtype == DOMINO_BF16 ? 2 : 4; }

int check_head(const domino_head* h) {
  if (!h) return DOMINO_ERR_NULL;
  if (h->dtype != DOMINO_F32 && h->dtype != DOMINO_BF16) return DOMINO_ERR_DTYPE;
  if (h->d <= 0 || h->vocab <= 0 || h->gru_hidden <= 0 || h->rank <= 0 || h->block <= 0) return DOMINO_ERR_SHAPE;
  if (h->d % 32 || h->gru_hidden % 32 || h->rank % 32) return DOMINO_ERR_SHAPE;
  if (h->block > kMaxBlock) return DOMINO_ERR_SHAPE;
  if (!h->lm_head || !h->embed || !h->w_ih || !h->w_hh || !h->w1 || !h->w2) return DOMINO_ERR_NULL;
  const void* mats[] = {h->lm_head, h->embed, h->w_ih, h->w_hh, h->w1, h->w2};
  for (const void* p : mats)
    if (!aligned16(p)) return DOMINO_ERR_ALIGN;
  if (h->gru_input_table && !aligned16(h->gru_input_table)) return DOMINO_ERR_ALIGN;
  const long es = elem_size(h->dtype);
  if ((long)h->d * es > kMaxRowBytes) return DOMINO_ERR_UNSUPPORTED;
  if (h->gru_hidden > kMaxGruHidden || h->rank > kMaxRank) return DOMINO_ERR_UNSUPPORTED;
  if (h->vocab > kMaxVocab) return DOMINO_ERR_UNSUPPORTED;
  return DOMINO_OK;
}

// ks: K-split of the W_ih e product, so that one 16-row tile of W_ih is shared
// by several waves; the slice must stay a multiple of 32 elements.
int gru_ksplit(int d) {
  for (int ks : {4, 2})
    if (d % (32 * ks) == 0) return ks;
  return 1;
}

static size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

WorkspaceLayout workspace_layout(const domino_head* h, int batch) {
  WorkspaceLayout w{};
  const size_t B = (size_t)batch, K = (size_t)h->block, H = (size_t)h->gru_hidden, r = (size_t)h->rank;
  const size_t ks = (size_t)gru_ksplit(h->d);
  size_t off = 0;
  w.keys = off;
  off += up256((K * B + 2) * sizeof(unsigned long long));  // keys + loop control words
  w.P = off;
  off += up256(B * K * r * sizeof(float));
  // K-slice partials of the hidden half of W1 h (bf16 heads): the single-block
  // loop and the per-position kernels add them up
  w.ppart = off;
  PSplit ps;
  if (h->dtype == DOMINO_BF16 && p_split_shape(h->d, h->rank, ps))
    off += up256((size_t)ps.S * B * K * r * sizeof(float));
  w.part_ih = off;
  off += up256(ks * B * 3 * H * sizeof(float));
  w.part_hh = off;
  off += up256(B * 3 * H * sizeof(float));
  w.u = off;
  off += up256(B * r * sizeof(float));
  w.states = off;
  off += up256(B * K * H * sizeof(float));
  // tagged exchange words of the persistent loop: partials, GRU state, u, keys,
  // each double-buffered by position parity
  const size_t multi = 2 * ((ks + 1) * B * 3 * H + B * H + B * r + (size_t)kMaxLoopWorkgroups * B);
  const size_t single = b1_exchange_words((int)H, (int)r, kMaxLoopWorkgroups);
  const size_t blocks = bn_exchange_words(batch, kMaxLoopWorkgroups, (int)H, (int)r);
  w.xwords = multi > single ? multi : single;
  if (blocks > w.xwords) w.xwords = blocks;
  w.xchg = off;
  off += up256(w.xwords * sizeof(unsigned long long));
  w.total = off;
  w.ks = (int)ks;
  return w;
}

bool forms_base_logits(const domino_head* h, int32_t batch) {
  return batch == 1 && h->dtype == DOMINO_BF16 && h->gru_input_table && h->block <= 16 &&
         (h->d == 2560 || h->d == 4096) && h->gru_hidden == 1024 && h->rank == 256;
}

int check_draft_io(const domino_head* h, int32_t batch, const void* hidden, const float* base_logits,
                   const int32_t* x_t, float temperature, int32_t* tokens, const float* logits,
                   const float* gru_states) {
  int st = check_head(h);
  if (st != DOMINO_OK) return st;
  if (batch < 0) return DOMINO_ERR_SHAPE;
  if (batch > kMaxBatch) return DOMINO_ERR_UNSUPPORTED;
  if (!std::isfinite(temperature) || temperature < 0.f) return DOMINO_ERR_ARG;
  if (batch == 0) return DOMINO_OK;
  if (!hidden || !x_t || !tokens) return DOMINO_ERR_NULL;
  if (!base_logits && !forms_base_logits(h, batch)) return DOMINO_ERR_UNSUPPORTED;
  if (!aligned16(hidden) || (base_logits && !aligned16(base_logits)) || !aligned16(tokens)) return DOMINO_ERR_ALIGN;
  if ((logits && !aligned16(logits)) || (gru_states && !aligned16(gru_states))) return DOMINO_ERR_ALIGN;
  return DOMINO_OK;
}

int check_draft_args(const domino_head* h, int32_t batch, const void* hidden, const float* base_logits,
                     const int32_t* x_t, float temperature, int32_t* tokens, const float* logits,
                     const float* gru_states, const void* workspace, size_t workspace_bytes) {
  int st = check_draft_io(h, batch, hidden, base_logits, x_t, temperature, tokens, logits, gru_states);
  if (st != DOMINO_OK || batch == 0) return st;
  const WorkspaceLayout w = workspace_layout(h, batch);
  if (!workspace) return DOMINO_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DOMINO_ERR_WORKSPACE;
  if (workspace_bytes < w.total) return DOMINO_ERR_WORKSPACE;
  return DOMINO_OK;
}

int check_base_args(const domino_head* h, int32_t batch, const void* hidden, const float* base_logits) {
  int st = check_head(h);
  if (st != DOMINO_OK) return st;
  if (batch < 0) return DOMINO_ERR_SHAPE;
  if (batch > kMaxBatch) return DOMINO_ERR_UNSUPPORTED;
  if (batch == 0) return DOMINO_OK;
  if (!hidden || !base_logits) return DOMINO_ERR_NULL;
  if (!aligned16(hidden) || !aligned16(base_logits)) return DOMINO_ERR_ALIGN;
  return DOMINO_OK;
}

int check_accept_args(int32_t batch, int32_t block, const int32_t* draft, const int32_t* target,
                      const int32_t* accept) {
  if (batch < 0 || block <= 0 || block > 1024) return DOMINO_ERR_SHAPE;
  if (batch == 0) return DOMINO_OK;
  if (!draft || !target || !accept) return DOMINO_ERR_NULL;
  return DOMINO_OK;
}

size_t base_draft_workspace_bytes(int32_t batch, int32_t block) {
  if (batch < 1 || batch > kMaxVerifyBatch || block < 1 || block > 1024) return 0;
  return ((size_t)batch * block * 8 + 255) & ~(size_t)255;
}

int check_base_draft_args(int32_t batch, int32_t block, int32_t vocab, const float* base_logits, float temperature,
                          const int32_t* tokens, const void* workspace, size_t workspace_bytes) {
  if (batch < 0 || batch > kMaxVerifyBatch || block < 1 || block > 1024 || vocab < 1 || vocab > kMaxVocab)
    return DOMINO_ERR_SHAPE;
  if (!(temperature >= 0.f) || !std::isfinite(temperature)) return DOMINO_ERR_ARG;
  if (batch == 0) return DOMINO_OK;
  if (!base_logits || !tokens) return DOMINO_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(base_logits) & 3u) return DOMINO_ERR_ALIGN;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      workspace_bytes < base_draft_workspace_bytes(batch, block))
    return DOMINO_ERR_WORKSPACE;
  return DOMINO_OK;
}

int check_loss_args(int32_t batch, int32_t block, int32_t vocab, const float* base_logits, const float* final_logits,
                    const int32_t* targets, float lambda, float gamma, const float* loss, const float* ce_base,
                    const float* ce_final, const float* grad_base, const float* grad_final, const void* workspace,
                    size_t workspace_bytes) {
  if (batch < 0 || batch > kMaxLossBatch || block < 1 || block > kMaxLossBlock || vocab < 1 || vocab > kMaxVocab)
    return DOMINO_ERR_SHAPE;
  if (!std::isfinite(lambda) || lambda < 0.f || lambda > 1.f) return DOMINO_ERR_ARG;
  if (!std::isfinite(gamma) || !(gamma > 0.f) || gamma > 1.f) return DOMINO_ERR_ARG;
  if (batch == 0) return DOMINO_OK;
  if (!base_logits || !final_logits || !targets || !loss) return DOMINO_ERR_NULL;
  for (const void* q : {(const void*)base_logits, (const void*)final_logits, (const void*)loss, (const void*)ce_base,
                        (const void*)ce_final, (const void*)grad_base, (const void*)grad_final})
    if (reinterpret_cast<uintptr_t>(q) & 3u) return DOMINO_ERR_ALIGN;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      workspace_bytes < loss_plan(batch, block, vocab).total)
    return DOMINO_ERR_WORKSPACE;
  return DOMINO_OK;
}

int check_backward_args(const domino_head* h, int32_t batch, const void* hidden, const float* gru_states,
                        const float* grad_final, const float* d_w2, const float* d_b2, const float* d_w1,
                        const float* d_b1, const float* d_states, const void* workspace, size_t workspace_bytes) {
  int st = check_head(h);
  if (st != DOMINO_OK) return st;
  if (batch < 0) return DOMINO_ERR_SHAPE;
  if (batch > kMaxBatch || h->rank > 512) return DOMINO_ERR_UNSUPPORTED;
  if (batch == 0) return DOMINO_OK;
  if (!hidden || !gru_states || !grad_final || !d_w2 || !d_w1) return DOMINO_ERR_NULL;
  if (!aligned16(hidden)) return DOMINO_ERR_ALIGN;
  for (const void* q : {(const void*)gru_states, (const void*)grad_final, (const void*)d_w2, (const void*)d_b2,
                        (const void*)d_w1, (const void*)d_b1, (const void*)d_states})
    if (reinterpret_cast<uintptr_t>(q) & 3u) return DOMINO_ERR_ALIGN;
  const BackwardPlan pl = backward_plan(batch * h->block, h->rank, h->vocab, h->dtype, h->d + h->gru_hidden, h->gru_hidden);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < pl.total)
    return DOMINO_ERR_WORKSPACE;
  return DOMINO_OK;
}

int check_gru_backward_args(const domino_head* h, int32_t batch, const int32_t* x_t, const int32_t* teacher,
                            const float* gru_states, const float* d_states, const float* d_w_ih,
                            const float* d_w_hh, const float* d_b_ih, const float* d_b_hh, const void* workspace,
                            size_t workspace_bytes) {
  int st = check_head(h);
  if (st != DOMINO_OK) return st;
  if (batch < 0) return DOMINO_ERR_SHAPE;
  if (batch > kMaxBatch) return DOMINO_ERR_UNSUPPORTED;
  if (batch == 0) return DOMINO_OK;
  if (!x_t || !teacher || !gru_states || !d_states || !d_w_ih || !d_w_hh) return DOMINO_ERR_NULL;
  for (const void* q : {(const void*)x_t, (const void*)teacher, (const void*)gru_states, (const void*)d_states,
                        (const void*)d_w_ih, (const void*)d_w_hh, (const void*)d_b_ih, (const void*)d_b_hh})
    if (reinterpret_cast<uintptr_t>(q) & 3u) return DOMINO_ERR_ALIGN;
  const GruBackwardPlan pl = gru_backward_plan(batch, h->block, h->d, h->gru_hidden, elem_size(h->dtype));
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < pl.total)
    return DOMINO_ERR_WORKSPACE;
  return DOMINO_OK;
}

int check_verify_args(int32_t batch, int32_t block, int32_t vocab, const float* target_logits,
                      const float* draft_logits, const int32_t* draft, float temperature, const int32_t* accept,
                      const int32_t* next_token, const void* workspace, size_t workspace_bytes) {
  if (batch < 0 || batch > kMaxVerifyBatch || block < 1 || block > kMaxVerifyBlock || vocab < 1 ||
      vocab > kMaxVocab)
    return DOMINO_ERR_SHAPE;
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return DOMINO_ERR_ARG;
  if (batch == 0) return DOMINO_OK;
  if (!target_logits || !draft_logits || !draft || !accept || !next_token) return DOMINO_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(target_logits) & 3u) || (reinterpret_cast<uintptr_t>(draft_logits) & 3u))
    return DOMINO_ERR_ALIGN;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      workspace_bytes < verify_plan(batch, block, vocab).total)
    return DOMINO_ERR_WORKSPACE;
  return DOMINO_OK;
}

}  // namespace domino

extern "C" const char* domino_status_string(int status) {
  switch (status) {
    case DOMINO_OK: return "ok";
    case DOMINO_ERR_NULL: return "a required pointer is NULL";
    case DOMINO_ERR_SHAPE: return "a size is out of range or not a multiple of 32";
    case DOMINO_ERR_DTYPE: return "unknown dtype code";
    case DOMINO_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case DOMINO_ERR_ARG: return "invalid scalar argument";
    case DOMINO_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case DOMINO_ERR_HIP: return "HIP runtime error";
    case DOMINO_ERR_UNSUPPORTED: return "request outside the library's limits";
    default: return "unknown status";
  }
}

extern "C" int domino_version(void) { return 100; }

extern "C" int domino_check_head(const domino_head* head) { return domino::check_head(head); }

extern "C" int domino_gru_table_size(const domino_head* head, size_t* bytes) {
  if (!bytes) return DOMINO_ERR_NULL;
  int st = domino::check_head(head);
  if (st != DOMINO_OK) return st;
  *bytes = (size_t)head->vocab * 3 * (size_t)head->gru_hidden * sizeof(float);
  return DOMINO_OK;
}

extern "C" int domino_workspace_size(const domino_head* head, int32_t batch, size_t* bytes) {
  if (!bytes) return DOMINO_ERR_NULL;
  int st = domino::check_head(head);
  if (st != DOMINO_OK) return st;
  if (batch < 0) return DOMINO_ERR_SHAPE;
  if (batch > domino::kMaxBatch) return DOMINO_ERR_UNSUPPORTED;
  *bytes = domino::workspace_layout(head, batch).total;
  return DOMINO_OK;
}
