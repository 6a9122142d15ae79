// sd_abi.hip -- the extern "C" entry points of libsd (declared in include/sd.h).
//
// Every entry point validates its scalars and required pointers before the
// first HIP call, sizes the workspace, and enqueues the kernels of its path on
// the caller's stream. It never allocates, frees or synchronises.
#include "sd.h"
#include "sd_internal.hpp"

#include <math.h>

#include <algorithm>
#include <mutex>

namespace {

constexpr int kMaxB = 1 << 20;
constexpr int kMaxV = (1 << 24) - 1;

bool bad_size(int B, int K_max, int V) {
    return B < 1 || B > kMaxB || K_max < 0 || K_max > SD_MAX_K || V < 1 || V > kMaxV;
}
bool bad_dtype(sd_dtype_t dt) { return dt != SD_F32 && dt != SD_BF16; }
bool topk_on(int top_k, int V) { return top_k >= 1 && top_k < V; }
// Base pointers the kernels read in 16-byte vectors (NULL passes: the
// separate NULL checks decide whether it is allowed).
bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

sd_status_t from_hip(hipError_t e) { return e == hipSuccess ? SD_OK : SD_EHIP; }

size_t chain_ws(int B, int K_max, int V, int dtype, float T, int top_k) {
    if (T == 0.0f) return sd::greedy_ws_bytes(B, K_max, V, dtype);
    if (topk_on(top_k, V)) return sd::chain_topk_ws_bytes(B, K_max, V, top_k);
    return sd::chain_full_ws_bytes(B, K_max, V, dtype);
}

}  // namespace

// Scratch space of sd_verify_chain_noalloc: a file-scope device array (each
// GPU holds its own copy). Host code never passes `scratch` itself to a kernel
// (on the host it only names the symbol): the per-device address from
// hipGetSymbolAddress is looked up once per device and used instead.
static __device__ __align__(256) unsigned char scratch[SD_NOALLOC_SCRATCH_BYTES];

namespace sd {
thread_local hipEvent_t PassTimer::start = nullptr;
thread_local hipEvent_t PassTimer::stop = nullptr;
}  // namespace sd

extern "C" {

int sd_abi_version(void) { return SD_ABI_VERSION; }

sd_status_t sd_time_next_stream_pass(void* start_event, void* stop_event) {
    sd::PassTimer::start = static_cast<hipEvent_t>(start_event);
    sd::PassTimer::stop = static_cast<hipEvent_t>(stop_event);
    return SD_OK;
}

const char* sd_status_str(int status) {
    switch (status) {
        case SD_OK: return "SD_OK";
        case SD_EINVAL: return "SD_EINVAL: invalid argument";
        case SD_EUNSUPPORTED: return "SD_EUNSUPPORTED: dtype/op combination not built";
        case SD_EWORKSPACE: return "SD_EWORKSPACE: workspace too small";
        case SD_EHIP: return "SD_EHIP: HIP launch failure";
        default: return "unknown sd status";
    }
}

sd_status_t sd_workspace_bytes(sd_op_t op, int32_t B, int32_t K_max, int32_t V, int32_t top_k,
                               int32_t N, size_t* bytes) {
    if (bytes == nullptr) return SD_EINVAL;
    *bytes = 0;
    switch (op) {
        case SD_OP_CHAIN:
            if (bad_size(B, K_max, V) || top_k < 0 || top_k > SD_MAX_TOPK) return SD_EINVAL;
            // the largest of the full-vocabulary, top-k and greedy layouts, either dtype
            {
                size_t m = sd::chain_full_ws_bytes(B, K_max, V, 0);
                m = std::max(m, sd::chain_full_ws_bytes(B, K_max, V, 1));
                if (topk_on(top_k, V)) m = std::max(m, sd::chain_topk_ws_bytes(B, K_max, V, top_k));
                m = std::max(m, sd::greedy_ws_bytes(B, K_max, V, 0));
                *bytes = std::max(m, sd::greedy_ws_bytes(B, K_max, V, 1));
            }
            return SD_OK;
        case SD_OP_GREEDY:
            if (bad_size(B, K_max, V)) return SD_EINVAL;
            *bytes = std::max(sd::greedy_ws_bytes(B, K_max, V, 0), sd::greedy_ws_bytes(B, K_max, V, 1));
            return SD_OK;
        case SD_OP_BUILD_TREE:
            if (B < 1 || B > kMaxB || K_max < 0 || K_max > SD_MAX_TREE_K || V < 1 || V > kMaxV ||
                N < 2 || N > SD_MAX_TREE_N)
                return SD_EINVAL;
            *bytes = sd::tree_build_ws_bytes(B, K_max, V, N);
            return SD_OK;
        case SD_OP_VERIFY_TREE:
            if (B < 1 || B > kMaxB || V < 1 || V > kMaxV || N < 2 || N > SD_MAX_TREE_N)
                return SD_EINVAL;
            *bytes = 0;   // the walk reads its rows on demand and keeps its state in LDS
            return SD_OK;
        case SD_OP_VERIFY_TREE_SAMPLED:
            if (B < 1 || B > kMaxB || V < 1 || V > kMaxV || N < 2 || N > SD_MAX_TREE_N || top_k < 0 ||
                top_k > SD_MAX_TOPK)
                return SD_EINVAL;
            *bytes = 0;   // both walks read their rows on demand and keep their state in LDS
            return SD_OK;
        case SD_OP_SELECT_LEN:
            if (B < 1 || B > kMaxB || K_max < 0 || K_max > SD_MAX_K) return SD_EINVAL;
            *bytes = 0;
            return SD_OK;
    }
    return SD_EINVAL;
}

}  // extern "C"

namespace {

// Argument checks shared by the chain entry points (no HIP call).
sd_status_t chain_args_status(const void* target_logits, const void* draft_logits, sd_dtype_t dtype,
                              const int32_t* draft_tokens, const float* uniforms, int32_t B,
                              int32_t K_max, int32_t V, float temperature, int32_t top_k,
                              const int32_t* accepted_len, const int32_t* next_token) {
    if (bad_size(B, K_max, V) || bad_dtype(dtype)) return SD_EINVAL;
    if (!(temperature >= 0.0f) || !isfinite(temperature)) return SD_EINVAL;
    if (top_k < 0 || top_k > SD_MAX_TOPK) return SD_EINVAL;
    if (!target_logits || !accepted_len || !next_token) return SD_EINVAL;
    if (misaligned(target_logits) || misaligned(draft_logits)) return SD_EINVAL;
    const bool greedy = temperature == 0.0f;
    if (K_max > 0 && !draft_tokens) return SD_EINVAL;
    if (!greedy && (!uniforms || (K_max > 0 && !draft_logits))) return SD_EINVAL;
    return SD_OK;
}

// sd_verify_chain and sd_verify_chain_capped: checks, then the path's launches.
sd_status_t verify_chain(const void* target_logits, const void* draft_logits, sd_dtype_t dtype,
                         const int32_t* draft_tokens, const float* uniforms, const int32_t* cu_draft,
                         const int32_t* cap, int32_t B, int32_t K_max, int32_t V, float temperature,
                         int32_t top_k, int32_t* accepted_len, int32_t* next_token,
                         int32_t* accepted_full, float* probs_out, float* resid_mass_out,
                         int32_t* seq_status, void* workspace, size_t workspace_bytes,
                         void* hip_stream) {
    const sd_status_t bad = chain_args_status(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                                              B, K_max, V, temperature, top_k, accepted_len, next_token);
    if (bad != SD_OK) return bad;
    if (!workspace || misaligned(workspace)) return SD_EINVAL;
    const bool greedy = temperature == 0.0f;
    const size_t need = chain_ws(B, K_max, V, (int)dtype, temperature, top_k);
    if (workspace_bytes < need) return SD_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (greedy)
        return from_hip(sd::launch_greedy(target_logits, (int)dtype, draft_tokens, cu_draft, B, K_max,
                                          V, accepted_len, next_token, seq_status, cap, accepted_full,
                                          workspace, st));
    sd::ChainArgs a;
    a.target = target_logits;
    a.draft = draft_logits;
    a.dtype = (int)dtype;
    a.tokens = draft_tokens;
    a.uniforms = uniforms;
    a.cu = cu_draft;
    a.B = B;
    a.K_max = K_max;
    a.V = V;
    a.temperature = temperature;
    a.top_k = top_k;
    a.accepted_len = accepted_len;
    a.next_token = next_token;
    a.probs_out = probs_out;
    a.resid_mass_out = resid_mass_out;
    a.seq_status = seq_status;
    a.cap = cap;
    a.accepted_full = accepted_full;
    a.ws = workspace;
    a.stream = st;
    if (topk_on(top_k, V)) return from_hip(sd::launch_chain_topk(a));
    return from_hip(sd::launch_chain_full(a));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch array, or nullptr on a HIP error.
void* scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

sd_status_t sd_verify_chain_noalloc(const void* target_logits, const void* draft_logits,
                                    sd_dtype_t dtype, const int32_t* draft_tokens,
                                    const float* uniforms, const int32_t* cu_draft, int32_t B,
                                    int32_t K_max, int32_t V, float temperature, int32_t top_k,
                                    int32_t* accepted_len, int32_t* next_token, float* probs_out,
                                    float* resid_mass_out, int32_t* seq_status, void* hip_stream) {
    // every argument check before the first HIP call (the scratch lookup)
    const sd_status_t bad = chain_args_status(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                                              B, K_max, V, temperature, top_k, accepted_len, next_token);
    if (bad != SD_OK) return bad;
    if (chain_ws(B, K_max, V, (int)dtype, temperature, top_k) > SD_NOALLOC_SCRATCH_BYTES)
        return SD_EWORKSPACE;
    void* ws = scratch_address();
    if (ws == nullptr) return SD_EHIP;
    return verify_chain(target_logits, draft_logits, dtype, draft_tokens, uniforms, cu_draft, nullptr,
                        B, K_max, V, temperature, top_k, accepted_len, next_token, nullptr, probs_out,
                        resid_mass_out, seq_status, ws, SD_NOALLOC_SCRATCH_BYTES, hip_stream);
}

sd_status_t sd_verify_chain(const void* target_logits, const void* draft_logits, sd_dtype_t dtype,
                            const int32_t* draft_tokens, const float* uniforms,
                            const int32_t* cu_draft, int32_t B, int32_t K_max, int32_t V,
                            float temperature, int32_t top_k, int32_t* accepted_len,
                            int32_t* next_token, float* probs_out, float* resid_mass_out,
                            int32_t* seq_status, void* workspace, size_t workspace_bytes,
                            void* hip_stream) {
    return verify_chain(target_logits, draft_logits, dtype, draft_tokens, uniforms, cu_draft, nullptr,
                        B, K_max, V, temperature, top_k, accepted_len, next_token, nullptr, probs_out,
                        resid_mass_out, seq_status, workspace, workspace_bytes, hip_stream);
}

sd_status_t sd_verify_chain_capped(const void* target_logits, const void* draft_logits,
                                   sd_dtype_t dtype, const int32_t* draft_tokens,
                                   const float* uniforms, const int32_t* k_cap, int32_t B,
                                   int32_t K_max, int32_t V, float temperature, int32_t top_k,
                                   int32_t* accepted_len, int32_t* next_token,
                                   int32_t* accepted_full, float* probs_out, float* resid_mass_out,
                                   int32_t* seq_status, void* workspace, size_t workspace_bytes,
                                   void* hip_stream) {
    if (!k_cap) return SD_EINVAL;
    return verify_chain(target_logits, draft_logits, dtype, draft_tokens, uniforms, nullptr, k_cap, B,
                        K_max, V, temperature, top_k, accepted_len, next_token, accepted_full,
                        probs_out, resid_mass_out, seq_status, workspace, workspace_bytes,
                        hip_stream);
}

sd_status_t sd_verify_greedy(const void* target_logits, sd_dtype_t dtype,
                             const int32_t* draft_tokens, const int32_t* cu_draft, int32_t B,
                             int32_t K_max, int32_t V, int32_t* accepted_len, int32_t* next_token,
                             int32_t* seq_status, void* workspace, size_t workspace_bytes,
                             void* hip_stream) {
    if (bad_size(B, K_max, V) || bad_dtype(dtype)) return SD_EINVAL;
    if (!target_logits || !accepted_len || !next_token || !workspace) return SD_EINVAL;
    if (misaligned(target_logits) || misaligned(workspace)) return SD_EINVAL;
    if (K_max > 0 && !draft_tokens) return SD_EINVAL;
    if (workspace_bytes < sd::greedy_ws_bytes(B, K_max, V, (int)dtype)) return SD_EWORKSPACE;
    return from_hip(sd::launch_greedy(target_logits, (int)dtype, draft_tokens, cu_draft, B, K_max, V,
                                      accepted_len, next_token, seq_status, nullptr, nullptr,
                                      workspace, static_cast<hipStream_t>(hip_stream)));
}

sd_status_t sd_build_tree(const float* marginals, int32_t B, int32_t K, int32_t V, int32_t N,
                          int32_t* node_token, int32_t* node_parent, int32_t* node_depth,
                          float* node_score, uint64_t* node_anc_mask, int32_t* n_nodes,
                          void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (B < 1 || B > kMaxB || K < 0 || K > SD_MAX_TREE_K || V < 1 || V > kMaxV || N < 2 ||
        N > SD_MAX_TREE_N)
        return SD_EINVAL;
    if ((K > 0 && !marginals) || !node_token || !node_parent || !node_depth || !node_score ||
        !node_anc_mask || !n_nodes)
        return SD_EINVAL;
    if (misaligned(marginals) || misaligned(workspace)) return SD_EINVAL;
    const size_t need = sd::tree_build_ws_bytes(B, K, V, N);
    if (need > 0 && !workspace) return SD_EINVAL;
    if (workspace_bytes < need) return SD_EWORKSPACE;
    return from_hip(sd::launch_tree_build(marginals, B, K, V, N, node_token, node_parent, node_depth,
                                          node_score, node_anc_mask, n_nodes, workspace,
                                          static_cast<hipStream_t>(hip_stream)));
}

sd_status_t sd_verify_tree(const void* target_logits, sd_dtype_t dtype, const int32_t* node_token,
                           const int32_t* node_parent, const int32_t* n_nodes, int32_t B, int32_t N,
                           int32_t V, int32_t* path_nodes, int32_t* accepted_len,
                           int32_t* next_token, void* workspace, size_t workspace_bytes,
                           void* hip_stream) {
    if (B < 1 || B > kMaxB || V < 1 || V > kMaxV || N < 2 || N > SD_MAX_TREE_N || bad_dtype(dtype))
        return SD_EINVAL;
    if (!target_logits || !node_token || !node_parent || !n_nodes || !path_nodes || !accepted_len ||
        !next_token)
        return SD_EINVAL;
    if (misaligned(target_logits)) return SD_EINVAL;
    (void)workspace;
    (void)workspace_bytes;
    return from_hip(sd::launch_tree_walk_rows(target_logits, (int)dtype, node_token, node_parent,
                                              n_nodes, nullptr, B, N, V, 0.0f, path_nodes,
                                              accepted_len, next_token, nullptr,
                                              static_cast<hipStream_t>(hip_stream)));
}

sd_status_t sd_verify_tree_sampled(const void* target_logits, sd_dtype_t dtype,
                                   const int32_t* node_token, const int32_t* node_parent,
                                   const int32_t* n_nodes, const float* uniforms, int32_t B,
                                   int32_t N, int32_t V, float temperature, int32_t top_k,
                                   int32_t* path_nodes, int32_t* accepted_len,
                                   int32_t* next_token, int32_t* seq_status, void* workspace,
                                   size_t workspace_bytes, void* hip_stream) {
    if (B < 1 || B > kMaxB || V < 1 || V > kMaxV || N < 2 || N > SD_MAX_TREE_N || bad_dtype(dtype))
        return SD_EINVAL;
    if (!isfinite(temperature) || temperature < 0.0f || top_k < 0 || top_k > SD_MAX_TOPK)
        return SD_EINVAL;
    if (!target_logits || !node_token || !node_parent || !n_nodes || !path_nodes || !accepted_len ||
        !next_token || (temperature > 0.0f && !uniforms))
        return SD_EINVAL;
    if (misaligned(target_logits)) return SD_EINVAL;
    (void)workspace;
    (void)workspace_bytes;
    const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (temperature > 0.0f && topk_on(top_k, V))
        return from_hip(sd::launch_tree_walk_topk(target_logits, (int)dtype, node_token, node_parent,
                                                  n_nodes, uniforms, B, N, V, temperature, top_k,
                                                  path_nodes, accepted_len, next_token, seq_status,
                                                  stream));
    return from_hip(sd::launch_tree_walk_rows(target_logits, (int)dtype, node_token, node_parent,
                                              n_nodes, uniforms, B, N, V, temperature, path_nodes,
                                              accepted_len, next_token, seq_status, stream));
}

sd_status_t sd_select_len(const float* conf, int32_t B, int32_t K_max, float cost_per_position,
                          int32_t* k_sel, float* expected_advance, int32_t* cu_sel,
                          void* hip_stream) {
    if (B < 1 || B > kMaxB || K_max < 0 || K_max > SD_MAX_K) return SD_EINVAL;
    if (!isfinite(cost_per_position)) return SD_EINVAL;
    if ((K_max > 0 && !conf) || !k_sel) return SD_EINVAL;
    return from_hip(sd::launch_select_len(conf, B, K_max, cost_per_position, nullptr, k_sel,
                                          expected_advance, cu_sel,
                                          static_cast<hipStream_t>(hip_stream)));
}

sd_status_t sd_select_len_table(const float* conf, int32_t B, int32_t K_max,
                                const float* cost_table, int32_t* k_sel, float* expected_advance,
                                int32_t* cu_sel, void* hip_stream) {
    if (B < 1 || B > kMaxB || K_max < 0 || K_max > SD_MAX_K) return SD_EINVAL;
    if ((K_max > 0 && (!conf || !cost_table)) || !k_sel) return SD_EINVAL;
    return from_hip(sd::launch_select_len(conf, B, K_max, 0.0f, cost_table, k_sel, expected_advance,
                                          cu_sel, static_cast<hipStream_t>(hip_stream)));
}

sd_status_t sd_expand_tree(int32_t* cand_parent, int32_t* cand_token, float* cand_prob,
                           float* cand_conf, int32_t* n_cand, const int32_t* expand_in,
                           int32_t* expand_out, const int32_t* child_token, const float* child_prob,
                           int32_t B, int32_t M, int32_t W, int32_t C, void* hip_stream) {
    if (B < 1 || B > kMaxB || M < 1 || M > SD_MAX_CANDIDATES || W < 1 || W > SD_MAX_EXPAND ||
        C < 1 || C > SD_MAX_CANDIDATES)
        return SD_EINVAL;
    if (!cand_parent || !cand_token || !cand_prob || !cand_conf || !n_cand || !expand_out ||
        !child_token || !child_prob)
        return SD_EINVAL;
    return from_hip(sd::launch_expand_tree(cand_parent, cand_token, cand_prob, cand_conf, n_cand,
                                           expand_in, expand_out, child_token, child_prob, B, M, W, C,
                                           static_cast<hipStream_t>(hip_stream)));
}

sd_status_t sd_stream_read(const void* data, size_t bytes, uint32_t* sink, int32_t n_blocks,
                           void* hip_stream) {
    if (!data || !sink || misaligned(data) || bytes % 16 != 0 || bytes == 0 || n_blocks < 1 ||
        n_blocks > (1 << 20))
        return SD_EINVAL;
    return from_hip(sd::launch_stream_read(data, (int64_t)bytes, sink, n_blocks,
                                           static_cast<hipStream_t>(hip_stream)));
}

sd_status_t sd_stream_read_rows(const void* data, size_t row_bytes, int32_t n_rows, size_t chunk_bytes,
                                uint32_t* sink, void* hip_stream) {
    if (!data || !sink || misaligned(data) || row_bytes == 0 || row_bytes % 16 != 0 || chunk_bytes == 0 ||
        chunk_bytes % 16 != 0 || n_rows < 1 || row_bytes > ((size_t)1 << 32))
        return SD_EINVAL;
    const size_t chunks = (row_bytes + chunk_bytes - 1) / chunk_bytes;
    if ((size_t)n_rows * chunks > ((size_t)1 << 24)) return SD_EINVAL;
    return from_hip(sd::launch_stream_read_rows(data, (int64_t)row_bytes, n_rows, (int64_t)chunk_bytes, sink,
                                                static_cast<hipStream_t>(hip_stream)));
}

sd_status_t sd_compact_kv(void* kv, int64_t row_bytes, int64_t n_rows, const int64_t* row_base,
                          const int32_t* path_nodes, const int32_t* accepted_len, int32_t B,
                          int32_t N, void* hip_stream) {
    if (B < 1 || B > kMaxB || N < 2 || N > SD_MAX_TREE_N) return SD_EINVAL;
    if (row_bytes < 16 || row_bytes % 16 != 0 || n_rows < 1) return SD_EINVAL;
    if (!kv || !row_base || !path_nodes || !accepted_len) return SD_EINVAL;
    if (misaligned(kv)) return SD_EINVAL;
    return from_hip(sd::launch_compact_kv(kv, row_bytes, n_rows, row_base, path_nodes, accepted_len, B,
                                          N, static_cast<hipStream_t>(hip_stream)));
}

sd_status_t sd_rerank_tree(const int32_t* cand_parent, const int32_t* cand_token,
                           const float* cand_prob, const int32_t* n_cand, int32_t B, int32_t M,
                           int32_t N, int32_t* node_token, int32_t* node_parent,
                           int32_t* node_depth, float* node_score, uint64_t* node_anc_mask,
                           int32_t* node_cand, int32_t* n_nodes, void* hip_stream) {
    if (B < 1 || B > kMaxB || M < 1 || M > SD_MAX_CANDIDATES || N < 2 || N > SD_MAX_TREE_N)
        return SD_EINVAL;
    if (!cand_parent || !cand_token || !cand_prob || !n_cand || !node_token || !node_parent ||
        !node_depth || !node_score || !node_anc_mask || !n_nodes)
        return SD_EINVAL;
    return from_hip(sd::launch_rerank_tree(cand_parent, cand_token, cand_prob, n_cand, B, M, N,
                                           node_token, node_parent, node_depth, node_score,
                                           node_anc_mask, node_cand, n_nodes,
                                           static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"
