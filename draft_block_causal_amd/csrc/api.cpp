// C ABI entry points of the Domino engine: validate on the host, then enqueue
// the kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kernels.h"
#include "validate.h"

namespace {

constexpr int kMaxDevices = 64;

int device_cu_count() {
  static int cu[kMaxDevices] = {0};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cu[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cu[dev] = n;
  }
  return cu[dev];
}

int hip_status(hipError_t e) { return e == hipSuccess ? DOMINO_OK : DOMINO_ERR_HIP; }

// DOMINO_LOOP selects the loop schedule: persistent (the cooperative kernel,
// B <= 32), multi (three kernels per position), blocks (the several-block
// on-chip loop also for two blocks); default: the library's choice.
int loop_mode() {
  const char* m = std::getenv("DOMINO_LOOP");
  if (!m) return 0;
  if (std::strcmp(m, "persistent") == 0) return 1;
  if (std::strcmp(m, "multi") == 0) return 2;
  if (std::strcmp(m, "blocks") == 0) return 3;
  if (std::strcmp(m, "perblock") == 0) return 4;  // never the several-block loop: one block at a time up to two
  return 0;
}

// DOMINO_DEBUG_SPIN_LIMIT=n sets the polls a wait of the on-chip loops makes
// before giving up (test hook: 0 makes every wait give up at its first check).
unsigned int spin_limit() {
  const char* m = std::getenv("DOMINO_DEBUG_SPIN_LIMIT");
  if (!m || !*m) return domino::kDefaultSpinLimit;
  char* end = nullptr;
  const unsigned long v = std::strtoul(m, &end, 10);
  if (end == m || *end != '\0' || v > domino::kDefaultSpinLimit) return domino::kDefaultSpinLimit;
  return (unsigned int)v;
}

}  // namespace

extern "C" int domino_base_logits(const domino_head* h, int32_t batch, const void* hidden, float* base_logits,
                                  void* stream) {
  int st = domino::check_base_args(h, batch, hidden, base_logits);
  if (st != DOMINO_OK || batch == 0) return st;
  const int num_cu = device_cu_count();
  if (num_cu <= 0) return DOMINO_ERR_HIP;
  const int M = batch * h->block;
  return hip_status(domino::launch_panel_gemm(h->dtype, hidden, h->d, M, h->lm_head, h->d, h->vocab, h->d,
                                              nullptr, base_logits, h->vocab, num_cu,
                                              static_cast<hipStream_t>(stream)));
}

extern "C" int domino_draft_block(const domino_head* h, int32_t batch, const void* hidden,
                                  const float* base_logits, const int32_t* x_t, const int32_t* teacher,
                                  float temperature, uint64_t seed, uint32_t offset, int32_t* tokens,
                                  float* logits, float* gru_states, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  int st = domino::check_draft_args(h, batch, hidden, base_logits, x_t, temperature, tokens, logits, gru_states,
                                    workspace, workspace_bytes);
  if (st != DOMINO_OK || batch == 0) return st;
  return domino::enqueue_draft_block(h, batch, hidden, base_logits, x_t, teacher, temperature, seed, offset, tokens,
                                     logits, gru_states, workspace, stream);
}

int domino::enqueue_draft_block(const domino_head* h, int32_t batch, const void* hidden, const float* base_logits,
                                const int32_t* x_t, const int32_t* teacher, float temperature, uint64_t seed,
                                uint32_t offset, int32_t* tokens, float* logits, float* gru_states, void* workspace,
                                void* stream) {
  const int num_cu = device_cu_count();
  if (num_cu <= 0) return DOMINO_ERR_HIP;
  const domino::WorkspaceLayout w = domino::workspace_layout(h, batch);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  domino::LoopArgs a{};
  a.dtype = h->dtype;
  a.B = batch;
  a.K = h->block;
  a.d = h->d;
  a.V = h->vocab;
  a.H = h->gru_hidden;
  a.r = h->rank;
  a.embed = h->embed;
  a.w_ih = h->w_ih;
  a.w_hh = h->w_hh;
  a.b_ih = h->b_ih;
  a.b_hh = h->b_hh;
  a.w1 = h->w1;
  a.b1 = h->b1;
  a.w2 = h->w2;
  a.b2 = h->b2;
  a.hidden = hidden;
  a.base = base_logits;
  a.lm_head = h->lm_head;
  a.x_t = x_t;
  a.teacher = teacher;
  a.sampled = temperature > 0.f ? 1 : 0;
  a.inv_temp = temperature > 0.f ? 1.0f / temperature : 0.f;
  a.seed = seed;
  a.offset = offset;
  a.tokens = tokens;
  a.logits = logits;
  a.states = gru_states ? gru_states : reinterpret_cast<float*>(ws + w.states);
  a.keys = reinterpret_cast<unsigned long long*>(ws + w.keys);
  a.P = reinterpret_cast<float*>(ws + w.P);
  a.ppart = reinterpret_cast<float*>(ws + w.ppart);
  a.part_ih = reinterpret_cast<float*>(ws + w.part_ih);
  a.part_hh = reinterpret_cast<float*>(ws + w.part_hh);
  a.u = reinterpret_cast<float*>(ws + w.u);
  a.table = h->gru_input_table;
  a.xpart = reinterpret_cast<unsigned long long*>(ws + w.xchg);
  a.xwords = w.xwords;
  a.max_wg = domino::kMaxLoopWorkgroups;
  a.ks = w.ks;
  a.num_cu = num_cu;
  a.call_status = reinterpret_cast<unsigned int*>(a.keys + (size_t)batch * h->block + 1);
  a.spin_limit = spin_limit();
  a.clear_words = batch * h->block + 2;
  if (!base_logits) {
    // the single-block loop forms the base logits itself; a device whose grid
    // it cannot hold (fewer than 200 compute units) has no other schedule for it
    const hipError_t e = domino::launch_draft_b1(a, static_cast<hipStream_t>(stream));
    return e == hipErrorNotSupported ? DOMINO_ERR_UNSUPPORTED : hip_status(e);
  }
  return hip_status(domino::launch_draft_loop(a, loop_mode(), static_cast<hipStream_t>(stream)));
}

extern "C" int domino_draft_status(const domino_head* h, int32_t batch, const void* workspace,
                                   size_t workspace_bytes, int32_t* status, void* stream) {
  int st = domino::check_head(h);
  if (st != DOMINO_OK) return st;
  if (batch < 1) return DOMINO_ERR_SHAPE;
  if (batch > domino::kMaxBatch) return DOMINO_ERR_UNSUPPORTED;
  if (!status) return DOMINO_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(status) & 3u) != 0) return DOMINO_ERR_ALIGN;
  const domino::WorkspaceLayout w = domino::workspace_layout(h, batch);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < w.total)
    return DOMINO_ERR_WORKSPACE;
  const unsigned char* word = static_cast<const unsigned char*>(workspace) + w.keys +
                              ((size_t)batch * h->block + 1) * sizeof(unsigned long long);
  return hip_status(hipMemcpyAsync(status, word, sizeof(int32_t), hipMemcpyDeviceToDevice,
                                   static_cast<hipStream_t>(stream)));
}

extern "C" int domino_prepare_gru_table(const domino_head* h, float* table, void* stream) {
  int st = domino::check_head(h);
  if (st != DOMINO_OK) return st;
  if (!table) return DOMINO_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(table) & 15u) != 0) return DOMINO_ERR_ALIGN;
  const int num_cu = device_cu_count();
  if (num_cu <= 0) return DOMINO_ERR_HIP;
  // T[v] = W_ih E[v] + b_ih for every vocabulary entry: C[V][3H] = E W_ih^T + b_ih
  return hip_status(domino::launch_panel_gemm(h->dtype, h->embed, h->d, h->vocab, h->w_ih, h->d,
                                              3 * h->gru_hidden, h->d, h->b_ih, table, 3 * h->gru_hidden,
                                              num_cu, static_cast<hipStream_t>(stream)));
}

extern "C" int domino_accept_len(int32_t batch, int32_t block, const int32_t* draft, const int32_t* target,
                                 int32_t* accept, void* stream) {
  int st = domino::check_accept_args(batch, block, draft, target, accept);
  if (st != DOMINO_OK || batch == 0) return st;
  return hip_status(domino::launch_accept_len(batch, block, draft, target, accept, static_cast<hipStream_t>(stream)));
}

extern "C" size_t domino_verify_workspace_size(int32_t batch, int32_t block, int32_t vocab) {
  if (batch < 1 || batch > domino::kMaxVerifyBatch || block < 1 || block > domino::kMaxVerifyBlock || vocab < 1 ||
      vocab > domino::kMaxVocab)
    return 0;
  return domino::verify_plan(batch, block, vocab).total;
}

extern "C" int domino_verify_sampled(int32_t batch, int32_t block, int32_t vocab, const float* target_logits,
                                     const float* draft_logits, const int32_t* draft, float temperature,
                                     uint64_t seed, uint32_t offset, int32_t* accept, int32_t* next_token,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  int st = domino::check_verify_args(batch, block, vocab, target_logits, draft_logits, draft, temperature, accept,
                                     next_token, workspace, workspace_bytes);
  if (st != DOMINO_OK || batch == 0) return st;
  return hip_status(domino::launch_verify_sampled(batch, block, vocab, target_logits, draft_logits, draft,
                                                  temperature, seed, offset, accept, next_token,
                                                  domino::verify_plan(batch, block, vocab), workspace,
                                                  static_cast<hipStream_t>(stream)));
}

extern "C" int domino_gru_backward_workspace_size(const domino_head* h, int32_t batch, size_t* bytes) {
  if (!bytes) return DOMINO_ERR_NULL;
  int st = domino::check_head(h);
  if (st != DOMINO_OK) return st;
  if (batch < 0) return DOMINO_ERR_SHAPE;
  if (batch > domino::kMaxBatch) return DOMINO_ERR_UNSUPPORTED;
  *bytes = batch == 0 ? 0
                      : domino::gru_backward_plan(batch, h->block, h->d, h->gru_hidden, domino::elem_size(h->dtype)).total;
  return DOMINO_OK;
}

extern "C" int domino_gru_backward(const domino_head* h, int32_t batch, const int32_t* x_t, const int32_t* teacher,
                                   const float* gru_states, const float* d_states, float* d_w_ih, float* d_w_hh,
                                   float* d_b_ih, float* d_b_hh, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  int st = domino::check_gru_backward_args(h, batch, x_t, teacher, gru_states, d_states, d_w_ih, d_w_hh, d_b_ih,
                                           d_b_hh, workspace, workspace_bytes);
  if (st != DOMINO_OK || batch == 0) return st;
  const int num_cu = device_cu_count();
  if (num_cu <= 0) return DOMINO_ERR_HIP;
  domino::GruBackwardArgs g{};
  g.dtype = h->dtype;
  g.B = batch;
  g.K = h->block;
  g.d = h->d;
  g.H = h->gru_hidden;
  g.V = h->vocab;
  g.embed = h->embed;
  g.w_ih = h->w_ih;
  g.w_hh = h->w_hh;
  g.b_ih = h->b_ih;
  g.b_hh = h->b_hh;
  g.x_t = x_t;
  g.teacher = teacher;
  g.states = gru_states;
  g.dg = d_states;
  g.d_w_ih = d_w_ih;
  g.d_w_hh = d_w_hh;
  g.d_b_ih = d_b_ih;
  g.d_b_hh = d_b_hh;
  g.workspace = workspace;
  g.plan = domino::gru_backward_plan(batch, h->block, h->d, h->gru_hidden, domino::elem_size(h->dtype));
  return hip_status(domino::launch_gru_backward(g, num_cu, static_cast<hipStream_t>(stream)));
}

extern "C" int domino_correction_backward_workspace_size(const domino_head* h, int32_t batch, size_t* bytes) {
  if (!bytes) return DOMINO_ERR_NULL;
  int st = domino::check_head(h);
  if (st != DOMINO_OK) return st;
  if (batch < 0) return DOMINO_ERR_SHAPE;
  if (batch > domino::kMaxBatch || h->rank > 512) return DOMINO_ERR_UNSUPPORTED;
  *bytes = batch == 0 ? 0 : domino::backward_plan(batch * h->block, h->rank, h->vocab, h->dtype, h->d + h->gru_hidden, h->gru_hidden).total;
  return DOMINO_OK;
}

extern "C" int domino_correction_backward(const domino_head* h, int32_t batch, const void* hidden,
                                          const float* gru_states, const float* grad_final, float* d_w2,
                                          float* d_b2, float* d_w1, float* d_b1, float* d_states, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  int st = domino::check_backward_args(h, batch, hidden, gru_states, grad_final, d_w2, d_b2, d_w1, d_b1, d_states,
                                       workspace, workspace_bytes);
  if (st != DOMINO_OK || batch == 0) return st;
  domino::BackwardArgs a{};
  a.dtype = h->dtype;
  a.R = batch * h->block;
  a.d = h->d;
  a.H = h->gru_hidden;
  a.r = h->rank;
  a.V = h->vocab;
  a.hidden = hidden;
  a.w1 = h->w1;
  a.b1 = h->b1;
  a.w2 = h->w2;
  a.states = gru_states;
  a.grad = grad_final;
  a.d_w2 = d_w2;
  a.d_b2 = d_b2;
  a.d_w1 = d_w1;
  a.d_b1 = d_b1;
  a.d_states = d_states;
  a.workspace = workspace;
  a.plan = domino::backward_plan(a.R, a.r, a.V, a.dtype, a.d + a.H, a.H);
  return hip_status(domino::launch_correction_backward(a, static_cast<hipStream_t>(stream)));
}

extern "C" size_t domino_curriculum_loss_workspace_size(int32_t batch, int32_t block, int32_t vocab) {
  if (batch < 1 || batch > domino::kMaxLossBatch || block < 1 || block > domino::kMaxLossBlock || vocab < 1 ||
      vocab > domino::kMaxVocab)
    return 0;
  return domino::loss_plan(batch, block, vocab).total;
}

extern "C" int domino_curriculum_loss(int32_t batch, int32_t block, int32_t vocab, const float* base_logits,
                                      const float* final_logits, const int32_t* targets, float lambda, float gamma,
                                      float* loss, float* ce_base, float* ce_final, float* grad_base,
                                      float* grad_final, void* workspace, size_t workspace_bytes, void* stream) {
  int st = domino::check_loss_args(batch, block, vocab, base_logits, final_logits, targets, lambda, gamma, loss,
                                   ce_base, ce_final, grad_base, grad_final, workspace, workspace_bytes);
  if (st != DOMINO_OK || batch == 0) return st;
  return hip_status(domino::launch_curriculum_loss(batch, block, vocab, base_logits, final_logits, targets, lambda,
                                                   gamma, loss, ce_base, ce_final, grad_base, grad_final,
                                                   domino::loss_plan(batch, block, vocab), workspace,
                                                   static_cast<hipStream_t>(stream)));
}

extern "C" size_t domino_base_draft_workspace_size(int32_t batch, int32_t block) {
  return domino::base_draft_workspace_bytes(batch, block);
}

extern "C" int domino_base_draft(int32_t batch, int32_t block, int32_t vocab, const float* base_logits,
                                 float temperature, uint64_t seed, uint32_t offset, int32_t* tokens, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  int st = domino::check_base_draft_args(batch, block, vocab, base_logits, temperature, tokens, workspace,
                                         workspace_bytes);
  if (st != DOMINO_OK || batch == 0) return st;
  return hip_status(domino::launch_base_draft(batch, block, vocab, base_logits, temperature, seed, offset, tokens,
                                              workspace, static_cast<hipStream_t>(stream)));
}

extern "C" int domino_debug_read_stream(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!sink || (bytes > 0 && !buf)) return DOMINO_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return DOMINO_ERR_ALIGN;
  if ((bytes & 15u) || bytes > ((size_t)1 << 40)) return DOMINO_ERR_SHAPE;
  return hip_status(domino::launch_read_stream(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

extern "C" int domino_debug_philox(uint64_t seed, uint32_t offset, int32_t b, int32_t pos, int32_t v0, int32_t n,
                                   uint32_t* out, void* stream) {
  if (n < 0 || n > (1 << 26) || b < 0 || pos < 0 || v0 < 0) return DOMINO_ERR_SHAPE;
  if (n == 0) return DOMINO_OK;
  if (!out) return DOMINO_ERR_NULL;
  return hip_status(domino::launch_debug_philox(seed, offset, b, pos, v0, n, out, static_cast<hipStream_t>(stream)));
}
