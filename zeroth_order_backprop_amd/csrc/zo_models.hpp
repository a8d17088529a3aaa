// Forward-only loss evaluation of the three model families, host side.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/zo.h"

namespace zo {

// Most losses one forward_loss call evaluates (probe-batched fused mode).
constexpr int kMaxEvalsPerCall = 64;

// Most tensors a model may have: a decoder of up to 255 layers.
constexpr int kMaxLayers = 255;
constexpr int kMaxTensors = 4 + 8 * kMaxLayers;

struct ModelView {
    zo_model_desc desc;
    void* params;
    void* workspace;
    size_t ws_bytes;
    const uint64_t* offsets;  // arena offset of each tensor, layout order (not owned)
    // The model's cache of captured decoder forwards (HIP graphs), created on
    // first use; null where the caller may not allocate: launches stay eager.
    void** graphs = nullptr;
    // The copies mode's device buffer (arena copies + grouped workspace) and
    // its size, grown on demand; null where the caller may not allocate.
    void** copies = nullptr;
    size_t* copies_bytes = nullptr;
};

// Releases a model's captured forwards (and their capture stream).
void decoder_graphs_free(void* cache);

zo_status model_check_shape(const zo_model_desc& d);
size_t model_workspace_bytes(const zo_model_desc& d);
// perts == nullptr: one loss at the stored weights into loss[0].
zo_status model_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n_perts,
                        double* loss, hipStream_t s);

// per family (zo_fp32_models.hip, zo_decoder.hip)
zo_status lsq_check(const zo_model_desc& d);
size_t lsq_workspace(const zo_model_desc& d);
zo_status lsq_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n, double* loss,
                      hipStream_t s);
zo_status mlp_check(const zo_model_desc& d);
size_t mlp_workspace(const zo_model_desc& d);
zo_status mlp_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n, double* loss,
                      hipStream_t s);
// split-perturbation (FedSPZO) step of the MLP, fused
zo_status mlp_split_check(const zo_model_desc& d, int p1, int ps);
zo_status mlp_split_step(const ModelView& m, const zo_batch& b, uint64_t seed, int p1, int ps, float eps, float lr,
                         double* losses, double* g1, double* g2, hipStream_t s);
// Dust (activation noise) step of the MLP
zo_status mlp_dust_check(const zo_model_desc& d, const zo_batch& b, int k1, int k2);
zo_status mlp_dust_step(const ModelView& m, const zo_batch& b, uint64_t seed, int k1, int k2, float sigma1,
                        float sigma2, float lr, double* losses, hipStream_t s);
zo_status decoder_check(const zo_model_desc& d);
size_t decoder_workspace(const zo_model_desc& d);
// Workspace of `groups` decoder evaluations side by side.
size_t decoder_group_workspace(const zo_model_desc& d, int groups);
// `groups` evaluations in one pass: group g at the weights params + g * gstride
// (arena copies, bf16 elements), workspace `ws` of decoder_group_workspace
// bytes; loss[g] = group g's mean loss.  batch * seq % 256 == 0 when groups > 1.
zo_status decoder_forward_groups(const ModelView& m, const zo_batch& b, const void* params, int groups,
                                 uint64_t gstride, void* ws, double* loss, hipStream_t s);
zo_status decoder_forward(const ModelView& m, const zo_batch& b, const zo_pert* perts, int n, double* loss,
                          hipStream_t s);

// kernel-level debug entry points (zo_decoder.hip)
zo_status debug_gemm_bf16(const void* A, const void* W, void* C, int M, int N, int K, int epi, hipStream_t s);
zo_status debug_attention(const void* qkv, void* out, int B, int S, int H, int dh, hipStream_t s);
zo_status debug_layernorm(const void* h, const void* g, const void* b, void* x, int rows, int d, hipStream_t s);

}  // namespace zo
