// Host-only validation and workspace layout (internal).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/domino.h"
#include "loss_plan.h"
#include "verify_plan.h"

namespace domino {

constexpr int kMaxBlock = 64;
constexpr int kMaxBatch = 128;
constexpr long kMaxRowBytes = 8192;
constexpr int kMaxGruHidden = 4096;
constexpr int kMaxRank = 1024;
constexpr int kMaxVocab = (1 << 24) - 1;  // the persistent loop's argmax keys hold a 24-bit index
constexpr int kMaxLoopWorkgroups = 1024;  // persistent loop grid cap (sizes the key exchange buffer)

struct WorkspaceLayout {
  size_t keys, P, ppart, part_ih, part_hh, u, states, xchg, total;
  size_t xwords;  // 64-bit words in the exchange region
  int ks;
};

int elem_size(int dtype);
int check_head(const domino_head* h);
int gru_ksplit(int d);
WorkspaceLayout workspace_layout(const domino_head* h, int batch);
// Whether a draft call of these shapes may leave the base logits to the
// single-block loop (base_logits == NULL): one block of at most 16 positions of
// a bf16 head with its GRU input table, d = 2560 or 4096, H = 1024, r = 256.
bool forms_base_logits(const domino_head* h, int32_t batch);
// Everything domino_draft_block checks except the workspace.
int check_draft_io(const domino_head* h, int32_t batch, const void* hidden, const float* base_logits,
                   const int32_t* x_t, float temperature, int32_t* tokens, const float* logits,
                   const float* gru_states);
int check_draft_args(const domino_head* h, int32_t batch, const void* hidden, const float* base_logits,
                     const int32_t* x_t, float temperature, int32_t* tokens, const float* logits,
                     const float* gru_states, const void* workspace, size_t workspace_bytes);
int check_base_args(const domino_head* h, int32_t batch, const void* hidden, const float* base_logits);
int check_accept_args(int32_t batch, int32_t block, const int32_t* draft, const int32_t* target,
                      const int32_t* accept);
int check_base_draft_args(int32_t batch, int32_t block, int32_t vocab, const float* base_logits, float temperature,
                          const int32_t* tokens, const void* workspace, size_t workspace_bytes);
size_t base_draft_workspace_bytes(int32_t batch, int32_t block);
int check_loss_args(int32_t batch, int32_t block, int32_t vocab, const float* base_logits, const float* final_logits,
                    const int32_t* targets, float lambda, float gamma, const float* loss, const float* ce_base,
                    const float* ce_final, const float* grad_base, const float* grad_final, const void* workspace,
                    size_t workspace_bytes);
int check_backward_args(const domino_head* h, int32_t batch, const void* hidden, const float* gru_states,
                        const float* grad_final, const float* d_w2, const float* d_b2, const float* d_w1,
                        const float* d_b1, const float* d_states, const void* workspace, size_t workspace_bytes);
int check_gru_backward_args(const domino_head* h, int32_t batch, const int32_t* x_t, const int32_t* teacher,
                            const float* gru_states, const float* d_states, const float* d_w_ih,
                            const float* d_w_hh, const float* d_b_ih, const float* d_b_hh, const void* workspace,
                            size_t workspace_bytes);
int check_verify_args(int32_t batch, int32_t block, int32_t vocab, const float* target_logits,
                      const float* draft_logits, const int32_t* draft, float temperature, const int32_t* accept,
                      const int32_t* next_token, const void* workspace, size_t workspace_bytes);

// Enqueues a draft call whose arguments passed check_draft_io, over a
// workspace of at least workspace_layout(h, batch).total bytes, 256-byte
// aligned (api.cpp).  Returns a domino_status.
int enqueue_draft_block(const domino_head* h, int32_t batch, const void* hidden, const float* base_logits,
                        const int32_t* x_t, const int32_t* teacher, float temperature, uint64_t seed,
                        uint32_t offset, int32_t* tokens, float* logits, float* gru_states, void* workspace,
                        void* stream);

}  // namespace domino
